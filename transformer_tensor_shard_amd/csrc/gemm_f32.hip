// f32 GEMM with the same fused epilogues as the bf16 kernel, for the
// full-precision path: C[M,N] = epi(A[M,K]·B[K,N] + bias[N]).
//
// gfx950's dense f32 rate is the vector-ALU rate (the chip has no f32
// matrix-core speedup), so this is a plain LDS-tiled FMA kernel: a 64x64 tile
// per 256-thread workgroup, 4x4 outputs per thread, K staged 16 at a time.
// Accumulation over k is in ascending k order per output, in f32.
#include "tp_kernels.h"

namespace tpk {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__device__ __forceinline__ float gelu_erf(float y) {
    return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
}

template <bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int64_t lda, const float* __restrict__ B, int64_t ldb,
    const float* __restrict__ bias, void* __restrict__ C, int64_t ldc, int M, int N, int K)
{
    __shared__ float As[TK][TM + 4];
    __shared__ float Bs[TK][TN + 4];
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        // 64x16 A tile and 16x64 B tile: 4 elements per thread each
        for (int e = threadIdx.x; e < TM * TK; e += 256) {
            const int r = e / TK, c = e % TK;
            const int gm = m0 + r, gk = k0 + c;
            As[c][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.0f;
        }
        for (int e = threadIdx.x; e < TK * TN; e += 256) {
            const int r = e / TN, c = e % TN;
            const int gk = k0 + r, gn = n0 + c;
            Bs[r][c] = (gk < K && gn < N) ? B[(int64_t)gk * ldb + gn] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < TK; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + ty + 16 * i;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx + 16 * j;
            if (col >= N) continue;
            float v = acc[i][j] + (bias ? bias[col] : 0.0f);
            if (GELU) v = gelu_erf(v);
            if (OUT_BF16)
                ((__bf16*)C)[(int64_t)row * ldc + col] = (__bf16)v;
            else
                ((float*)C)[(int64_t)row * ldc + col] = v;
        }
    }
}

}  // namespace

hipError_t gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                    const float* bias, void* C, int64_t ldc,
                    int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                    hipStream_t stream)
{
    const dim3 grid((unsigned)((N + TN - 1) / TN), (unsigned)((M + TM - 1) / TM)), block(256);
    if (out_bf16 && gelu)
        hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, block, 0, stream,
                           A, lda, B, ldb, bias, C, ldc, (int)M, (int)N, (int)K);
    else if (out_bf16)
        hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, block, 0, stream,
                           A, lda, B, ldb, bias, C, ldc, (int)M, (int)N, (int)K);
    else if (gelu)
        hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, block, 0, stream,
                           A, lda, B, ldb, bias, C, ldc, (int)M, (int)N, (int)K);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, block, 0, stream,
                           A, lda, B, ldb, bias, C, ldc, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace tpk
