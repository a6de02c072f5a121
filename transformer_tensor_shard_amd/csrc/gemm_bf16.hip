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
//    the next step's loads in flight while the MFMAs of this one run;
//  * global -> LDS traffic uses the gfx950 direct-to-LDS 16-byte buffer loads
//    (no staging registers, no LDS write instructions); lanes past M, N or K
//    are pushed out of the buffer's range, for which the load writes zeros;
//  * the 16-wide k-step fragments are double-buffered in registers so LDS
//    reads for the next k-step overlap the MFMAs of this one;
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

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// One k-step: 16 MFMAs with the next k-step's 12 LDS reads (4 A, 8 B) issued
// two at a time between the first six, so they land long before use.
__device__ __forceinline__ void sched_kstep() {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 10, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// The k-step after the barrier also issues the 16 direct-to-LDS loads of the
// tile after next.
__device__ __forceinline__ void sched_kstep_dma() {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 6, 0);
    __builtin_amdgcn_sched_barrier(0);
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
    // Two stages as two separate LDS objects: every access below names its
    // stage statically, which lets the compiler see that reads of one stage
    // do not depend on the direct-to-LDS loads still landing in the other.
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;

    const __bf16* a_tile = A + (int64_t)m0 * lda;
    const __bf16* b_tile = B + n0;

    // ---- global -> LDS: direct (DMA) 16-byte buffer loads ---------------------
    // A buffer_load_dwordx4 ... lds instruction writes 64 lanes x 16 B = 1 KiB
    // contiguously in LDS (lane l at M0 + 16 l), so the swizzled LDS layout is
    // produced by choosing which global unit each lane fetches.  Wave w fills
    // bytes [8 KiB w, 8 KiB w + 8 KiB) of each tile with 8 instructions:
    //   A: instruction j, lane l -> LDS row 64w + 8j + l/8, physical unit l%8
    //   B: instruction j, lane l -> LDS row 16w + 2j + l/32, physical unit l%32
    // and the logical unit is the physical one XOR the row's swizzle.
    unsigned a_off[8], b_off[8];
    int a_kcol[8], b_krow[8];
    bool a_row_ok[8], b_col_ok[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 64 * wid + 8 * j + (lane >> 3);
        const int u = (lane & 7) ^ ((r >> 1) & 7);
        a_row_ok[j] = (m0 + r) < M;
        a_kcol[j] = u * 8;
        a_off[j] = (unsigned)(r * lda + u * 8) * 2u;
        const int kr = 16 * wid + 2 * j + (lane >> 5);
        const int ub = (lane & 31) ^ ((kr & 3) << 2);
        b_col_ok[j] = (n0 + ub * 8) < N;
        b_krow[j] = kr;
        b_off[j] = (unsigned)(kr * ldb + ub * 8) * 2u;
    }
    // Lanes past M, N or K fetch nothing and the DMA writes zeros for them, so
    // ragged tails (and a tile index past the last one) need no branch.
    auto dma_tile = [&](int k0, char* stage) {
        const __amdgpu_buffer_rsrc_t ar = make_rsrc(a_tile + k0);
        const __amdgpu_buffer_rsrc_t br = make_rsrc(b_tile + (int64_t)k0 * ldb);
        char* sa = stage + wid * 8192;
        char* sb = stage + A_BYTES + wid * 8192;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = a_row_ok[j] && (k0 + a_kcol[j]) < K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, LDS_PTR(void, sa + j * 1024), 16,
                                                     ok ? a_off[j] : OOB, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = b_col_ok[j] && (k0 + b_krow[j]) < K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(br, LDS_PTR(void, sb + j * 1024), 16,
                                                     ok ? b_off[j] : OOB, 0, 0, 0);
        }
    };
    const int nk = (K + BK - 1) / BK;

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
    const int b_row = (g >> 1) * 8 + (gi >> 2);       // + 16*kk + 4*half
    unsigned b_rd[4];
#pragma unroll
    for (int nj = 0; nj < 4; ++nj) {
        const int col = wn * 128 + nj * 32 + (g & 1) * 16 + 4 * (gi & 3);
        const int unit = col >> 3;
        b_rd[nj] = A_BYTES + b_row * 512 + ((unit ^ ((b_row & 3) << 2)) << 4) + (col & 7) * 2;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    bf16x8 fa[2][4], fb[2][4];
    auto load_frags = [&](bf16x8 (&a)[4], bf16x8 (&b)[4], const char* base, int kk) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) a[mi] = *(const bf16x8*)(base + a_rd[kk] + mi * 32 * 128);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
            const char* p = base + b_rd[nj] + kk * 16 * 512;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p + 4 * 512));
            b[nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto mfmas = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[4]) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nj], acc[mi][nj], 0, 0, 0);
    };

    // ---- main loop: tile kt+1 is in flight into the other stage while tile kt
    // is multiplied; k-step fragments are double-buffered in registers; the
    // barrier that publishes tile kt+1 sits before the last k-step so that the
    // next tile's first fragments (and tile kt+2's loads) issue under the last
    // 16 MFMAs.  Scheduling groups pin the interleave: each k-step issues the
    // next k-step's 12 LDS reads between its first MFMAs.
    dma_tile(0, lds0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA has landed
    __syncthreads();
    dma_tile(BK, lds1);
    load_frags(fa[0], fb[0], lds0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // one K tile: three k-steps on `cur`, publish `nxt`, refill `cur` with the
    // tile after next, last k-step while the next tile's first fragments load
    auto tile = [&](const char* cur_c, char* cur, const char* nxt, int k_next2) {
        load_frags(fa[1], fb[1], cur_c, 1);
        mfmas(fa[0], fb[0]);
        sched_kstep();
        load_frags(fa[0], fb[0], cur_c, 2);
        mfmas(fa[1], fb[1]);
        sched_kstep();
        load_frags(fa[1], fb[1], cur_c, 3);
        mfmas(fa[0], fb[0]);
        sched_kstep();
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                            // next tile visible; `cur` free
        dma_tile(k_next2, cur);                     // all lanes masked past the last tile
        load_frags(fa[0], fb[0], nxt, 0);
        mfmas(fa[1], fb[1]);
        sched_kstep_dma();
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        tile(lds0, lds0, lds1, (kt + 2) * BK);
        tile(lds1, lds1, lds0, (kt + 3) * BK);
    }
    if (kt < nk) tile(lds0, lds0, lds1, (kt + 2) * BK);
    // the (masked, zero-writing) loads issued for the tiles past the end must
    // land before this workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);

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
