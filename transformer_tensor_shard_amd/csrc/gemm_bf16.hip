// bf16 x bf16 -> f32-accumulate GEMM for gfx950 (CDNA4) with fused epilogues.
//
// Computes C[M,N] = epi(A[M,K]·B[K,N] + bias[N]) for row-major A (the
// activations X, K contiguous) and row-major B (a weight in the [in, out]
// layout of the Megatron explainer's Y = X @ W, N contiguous).  This is the
// product behind the column-parallel layer (epilogue: + bias, exact-erf GeLU,
// store bf16: "图解Transformer并行计算" §2.1, Y'_i = GeLU(X·A_i)) and the
// row-parallel layer (epilogue: store the f32 partial, §2.1 Z_i = Y'_i·B_i).
//
// Design (one 256x256 output tile per workgroup, 4 waves of 64 lanes):
//  * each wave owns a 128x128 sub-tile = 4x4 MFMA 32x32x16 bf16 blocks
//    (256 f32 accumulators per lane, held in the unified VGPR/AGPR file);
//  * K advances in 64-wide steps; the A and B tiles of a step (32 KiB each)
//    are staged in LDS, double-buffered (128 KiB of the 160 KiB per CU), with
//    the next step's global loads in flight while the MFMAs of this one run;
//  * global loads are 16-byte buffer loads whose out-of-range lanes return 0
//    (ragged M, N and K tails need no branches in the loop);
//  * the A operand (K contiguous) is read with 16-byte LDS reads; the B
//    operand (N contiguous) is read with the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16), which hands each lane 4 consecutive K values of
//    one N column -- the layout the MFMA B operand wants -- so B is never
//    transposed in memory;
//  * both LDS tiles are XOR-swizzled in 16-byte units so that the writes, the
//    16-byte A reads and the transpose B reads each touch all 64 LDS banks
//    without conflicts;
//  * tiles are renumbered so that consecutive tiles land on the same XCD
//    (workgroups are dealt round-robin to the 8 XCDs, each with its own L2)
//    and walk the output in groups of 8 tile-rows.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int A_BYTES = BM * BK * 2;          // 32 KiB
constexpr int B_BYTES = BK * BN * 2;          // 32 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 8;
constexpr unsigned OOB = 0x80000000u;         // any offset >= num_records reads 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    // raw buffer, stride 0, num_records just below 2 GiB; word3 = gfx9 format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             0x7ffffff0, 0x00020000);
}

__device__ __forceinline__ float gelu_erf(float y) {
    return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f));
}

// Map a linear workgroup id to (tile_m, tile_n): first make the ids of one XCD
// contiguous, then walk GROUP_M tile-rows at a time.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int xcd = pid & 7, local = pid >> 3;
    const int per = ntiles >> 3, rem = ntiles & 7;
    const int id = (xcd < rem) ? xcd * (per + 1) + local
                               : rem * (per + 1) + (xcd - rem) * per + local;
    const int width = GROUP_M * tiles_n;
    const int group = id / width;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_group = id - group * width;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

template <bool OUT_BF16, bool GELU>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(
    const __bf16* __restrict__ A, int64_t lda, const __bf16* __restrict__ B, int64_t ldb,
    const float* __restrict__ bias, void* __restrict__ C, int64_t ldc,
    int M, int N, int K, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE_BYTES];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;

    // ---- global -> LDS copy assignment -------------------------------------
    // A tile: 256 rows x 8 units of 16 B; thread owns unit (tid & 7) of rows
    // (tid >> 3) + 32 i.  B tile: 64 rows x 32 units; thread owns unit
    // (tid & 31) of rows (tid >> 5) + 8 i.
    const int a_unit = tid & 7, a_row0 = tid >> 3;
    const int b_unit = tid & 31, b_row0 = tid >> 5;
    unsigned a_voff[8], b_voff[8];
    bool a_row_ok[8];
    unsigned a_lds[8], b_lds[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = a_row0 + 32 * i;
        a_row_ok[i] = (m0 + r) < M;
        a_voff[i] = (unsigned)(r * lda + a_unit * 8) * 2u;
        a_lds[i] = r * 128 + ((a_unit ^ ((r >> 1) & 7)) << 4);
        const int kr = b_row0 + 8 * i;
        b_voff[i] = (unsigned)(kr * ldb + b_unit * 8) * 2u;
        b_lds[i] = A_BYTES + kr * 512 + ((b_unit ^ ((kr & 3) << 2)) << 4);
    }
    const bool b_col_ok = (n0 + b_unit * 8) < N;

    const __bf16* a_tile = A + (int64_t)m0 * lda;
    const __bf16* b_tile = B + n0;

    u32x4 ra[8], rb[8];
    auto load_tiles = [&](int k0) {
        const __amdgpu_buffer_rsrc_t ar = make_rsrc(a_tile + k0);
        const __amdgpu_buffer_rsrc_t br = make_rsrc(b_tile + (int64_t)k0 * ldb);
        const bool a_k_ok = (k0 + a_unit * 8) < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const unsigned off = (a_row_ok[i] && a_k_ok) ? a_voff[i] : OOB;
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(ar, off, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = b_col_ok && (k0 + b_row0 + 8 * i) < K;
            rb[i] = __builtin_amdgcn_raw_buffer_load_b128(br, ok ? b_voff[i] : OOB, 0, 0);
        }
    };
    auto store_tiles = [&](int stage) {
        char* base = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4*)(base + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4*)(base + b_lds[i]) = rb[i];
    };

    // ---- LDS -> register operand addresses ----------------------------------
    // A operand of MFMA 32x32x16: lane holds row (lane & 31), K values
    // 8*(lane >> 5) .. +7 of the 16-wide k-step.
    const int a_r = wm * 128 + (lane & 31);
    const int a_swz = (a_r >> 1) & 7;
    unsigned a_rd[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        a_rd[kk] = a_r * 128 + (((kk * 2 + (lane >> 5)) ^ a_swz) << 4);
    // B operand via transpose reads: a group of 16 lanes reads a 4(K) x 16(N)
    // block; lane i of the group addresses row (i >> 2), columns 4*(i & 3)..+3
    // and receives column i, rows 0..3.  Groups 0/1 cover N columns 0-15 /
    // 16-31 of K rows 0-7, groups 2/3 the same columns of K rows 8-15.
    const int g = lane >> 4, gi = lane & 15;
    const int b_krow = (g >> 1) * 8 + (gi >> 2);       // + 16*kk + 4*half
    unsigned b_rd[4];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        const int col = wn * 128 + nj * 32 + (g & 1) * 16 + 4 * (gi & 3);
        const int unit = col >> 3;
        b_rd[nj] = A_BYTES + b_krow * 512 + ((unit ^ ((b_krow & 3) << 2)) << 4) + (col & 7) * 2;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (K + BK - 1) / BK;
    load_tiles(0);
    store_tiles(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool has_next = (kt + 1) < nk;
        if (has_next) load_tiles((kt + 1) * BK);
        const char* base = lds + cur * STAGE_BYTES;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = *(const bf16x8*)(base + a_rd[kk] + mi * 32 * 128);
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) {
                const char* p = base + b_rd[nj] + kk * 16 * 512;
                bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p));
                bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p + 4 * 512));
                bfr[nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int nj = 0; nj < 4; ++nj)
                    acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[nj],
                                                                          acc[mi][nj], 0, 0, 0);
        }
        if (has_next) store_tiles(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds column (lane & 31) and rows
    // 8*(r >> 2) + 4*(lane >> 5) + (r & 3) of each 32x32 block.
    const int row_base = m0 + wm * 128 + 4 * (lane >> 5);
    const int col_base = n0 + wn * 128 + (lane & 31);
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        const int col = col_base + nj * 32;
        if (col >= N) continue;
        const float bv = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row_base + mi * 32 + 8 * (r >> 2) + (r & 3);
                if (row >= M) continue;
                float v = acc[mi][nj][r] + bv;
                if (GELU) v = gelu_erf(v);
                if (OUT_BF16)
                    ((__bf16*)C)[(int64_t)row * ldc + col] = (__bf16)v;
                else
                    ((float*)C)[(int64_t)row * ldc + col] = v;
            }
        }
    }
}

}  // namespace

hipError_t gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                     const float* bias, void* C, int64_t ldc,
                     int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                     hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid(tiles_m * tiles_n), block(NTHREADS);
    const __bf16* a = (const __bf16*)A;
    const __bf16* b = (const __bf16*)B;
    if (out_bf16 && gelu)
        hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, block, 0, stream,
                           a, lda, b, ldb, bias, C, ldc, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    else if (out_bf16)
        hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), grid, block, 0, stream,
                           a, lda, b, ldb, bias, C, ldc, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    else if (gelu)
        hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), grid, block, 0, stream,
                           a, lda, b, ldb, bias, C, ldc, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, block, 0, stream,
                           a, lda, b, ldb, bias, C, ldc, (int)M, (int)N, (int)K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace tpk
