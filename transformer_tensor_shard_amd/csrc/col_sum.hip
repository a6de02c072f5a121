// Column sums of a bf16 matrix into f32: the bias gradient of a linear layer,
// da = Σ_rows dY ("图解Transformer并行计算" §2.2: each rank computes the
// gradients of its own parameters; a bias added to every token row receives
// the sum of that row-wise gradient over all tokens).
//
// HBM-bound and deterministic, in two launches:
//  * stage 1: workgroup (x, y) sums rows [256 y, 256 y + 256) of the 512
//    columns starting at 512 x; its 4 waves take every 4th row (one 1 KiB
//    row segment per wave and load, 16-byte loads), and their 4 sums are
//    added in wave order into part[y][col];
//  * stage 2: one thread per column adds part[0..chunks)[col] in order.
// The order of every addition is fixed by the shape alone, so the result is
// bitwise reproducible.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CS_COLS = 512;     // columns per workgroup: 64 lanes x 8

__global__ __launch_bounds__(256) void col_sum_partial_kernel(const __bf16* __restrict__ X,
                                                              int64_t ldx, int64_t M, int64_t N,
                                                              float* __restrict__ part)
{
    __shared__ float red[4][CS_COLS];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * CS_COLS + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * kColSumRows;
    const int64_t r1 = min(M, r0 + kColSumRows);
    float acc[8] = {};
    if (c0 < N) {                      // N % 8 == 0: the whole unit is in range
#pragma unroll 4
        for (int64_t r = r0 + w; r < r1; r += 4) {
            const bf16x8 v = *(const bf16x8*)(X + r * ldx + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
        }
    }
    *(f32x4*)&red[w][lane * 8] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)&red[w][lane * 8 + 4] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    for (int c = threadIdx.x; c < CS_COLS; c += 256) {
        const int64_t col = (int64_t)blockIdx.x * CS_COLS + c;
        if (col < N) part[blockIdx.y * N + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
}

__global__ __launch_bounds__(256) void col_sum_final_kernel(const float* __restrict__ part,
                                                            int chunks, int64_t N,
                                                            float* __restrict__ out)
{
    const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (col >= N) return;
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * N + col];
    out[col] = s;
}

}  // namespace

int64_t col_sum_chunks(int64_t M) { return (M + kColSumRows - 1) / kColSumRows; }

hipError_t col_sum(float* out, const void* X, int64_t ldx, int64_t M, int64_t N, float* part,
                   hipStream_t stream)
{
    const int chunks = (int)col_sum_chunks(M);
    const dim3 g1((unsigned)((N + CS_COLS - 1) / CS_COLS), (unsigned)chunks);
    hipLaunchKernelGGL(col_sum_partial_kernel, g1, dim3(256), 0, stream, (const __bf16*)X, ldx,
                       M, N, part);
    hipLaunchKernelGGL(col_sum_final_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0,
                       stream, (const float*)part, chunks, N, out);
    return hipGetLastError();
}

}  // namespace tpk
