// bf16 x bf16 -> f32-accumulate GEMM for gfx950 (CDNA4) with fused epilogues.
//
// Computes C[M,N] = epi(A[M,K]·B[K,N] + bias[N]) for row-major A (the
// activations X, K contiguous) and row-major B (a weight in the [in, out]
// layout of the Megatron explainer's Y = X @ W, N contiguous).  This is the
// product behind the column-parallel layer (epilogue: + bias, GeLU, store
// bf16: "图解Transformer并行计算" §2.1, Y'_i = GeLU(X·A_i)) and the
// row-parallel layer (epilogue: store the f32 partial, §2.1 Z_i = Y'_i·B_i).
//
// Design: one 256x256 output tile per workgroup of 8 waves (two per SIMD).
//  * wave w owns a 128x64 sub-tile: rows 128*((w&3)>>1), columns
//    128*(w&1) + 64*(w>>2); that is 8x4 MFMA 16x16x32 bf16 blocks with 128
//    f32 accumulators per lane.  The two waves on a SIMD (w and w+4) take the
//    two 64-column halves of one 128x128 quadrant, so while one of them waits
//    on memory the other keeps the SIMD's matrix core busy.  (16x16x32 rather
//    than 32x32x16: with two waves per SIMD it sustains ~10% more MFMA
//    throughput on MI355X under the power limit, measured, for the same
//    operand bytes per FLOP);
//  * K advances in 64-wide steps; the A and B tiles of a step (32 KiB each)
//    are staged in LDS, double-buffered (128 KiB of the 160 KiB per CU);
//  * global -> LDS traffic uses the gfx950 direct-to-LDS 16-byte buffer loads
//    (no staging registers, no LDS write instructions).  Per-lane offsets are
//    loop-invariant and only the scalar base of the buffer resource moves per
//    K step, so issuing a tile's loads costs no vector-ALU work; lanes whose
//    row (A) or column group (B) lies past M or N get an offset beyond the
//    buffer's range, for which the load writes zeros;
//  * operands of the next 32-wide k-step are read from LDS while this one's
//    32 MFMAs run: the B fragments into a second buffer, each A fragment into
//    its own registers right after its last MFMA (64 operand VGPRs, not 96);
//  * the A operand (K contiguous) is read with 16-byte LDS reads; the B
//    operand (N contiguous) with the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16), which hands each lane 4 consecutive K values of one
//    N column -- the layout the MFMA B operand wants -- so B is never
//    transposed in memory;
//  * both LDS tiles are XOR-swizzled in 16-byte units so that the DMA writes,
//    the 16-byte A reads and the transpose B reads are free of bank conflicts;
//  * tiles are renumbered so that consecutive tiles land on the same XCD
//    (workgroups are dealt round-robin to the 8 XCDs, each with its own L2)
//    and walk the output in groups of 4 tile-rows; a grouped launch whose
//    groups share the activations walks row bands across all groups;
//  * epilogue: the tile is staged through the (then idle) LDS and written with
//    16-byte row-contiguous stores: one pass for a bf16 tile, two for f32.
//
// Measured on MI355X the kernel is bound by the chip's power limit rather than
// by any one unit: sustained MFMA issue alone pulls the shader clock from 2.4
// to about 1.6-1.8 GHz, and every byte moved (HBM, L2, LDS) competes for the
// same budget.
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NWAVES = 8, NTHREADS = NWAVES * 64;
constexpr int A_BYTES = BM * BK * 2;          // 32 KiB
constexpr int B_BYTES = BK * BN * 2;          // 32 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 4;
constexpr unsigned OOB = 0x80000000u;         // any offset >= num_records reads 0
constexpr int NI = 8, NJ = 4;                 // 16x16 MFMA blocks per wave (rows, cols)
constexpr int LOADS = 4;                      // A (and B) loads per wave per K tile

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// One k-step of a wave: 8 MFMAs with the next k-step's 8 LDS reads issued
// one after each of the first 8 MFMAs, and V direct-to-LDS loads spread
// evenly between them.
#ifndef DSP
#define DSP 1
#endif
// One 32-wide k-step of a wave: 32 MFMAs (A block mi = I/4 against the 4 B
// blocks); the next k-step's 8 B reads go out after the first 8 MFMAs and
// each A block's reload right after its last MFMA; V direct-to-LDS loads are
// spread one per 32/V MFMAs.
template <int V, int I>
__device__ __forceinline__ void sched_step() {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    constexpr int nds = (I < 8 ? 1 : 0) + (I % 4 == 3 ? 1 : 0);
    if constexpr (nds > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, nds, 0);
    constexpr int nv = ((I + 1) * V) / 32 - (I * V) / 32;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, nv, 0);
    if constexpr (I + 1 < 32) sched_step<V, I + 1>();
}
template <int V>
__device__ __forceinline__ void sched_kstep() {
    sched_step<V, 0>();
    __builtin_amdgcn_sched_barrier(0);
}

// GeLU(x) = x·Φ(x), Φ(x) = 1 - erfc(x/√2)/2 for x >= 0 and erfc(|x|/√2)/2
// below, with erfc from Abramowitz & Stegun, Handbook of Mathematical
// Functions, eq. 7.1.26 (|error| <= 1.5e-7).  Branch-free; in f32 the result
// is within 4.3e-7 of the exact-erf GeLU over the whole real line, the same
// bound as x/2·(1 + erff(x/√2)) evaluated in f32.
__device__ __forceinline__ float gelu(float x) {
    const float t = fabsf(x) * 0.70710678118654752f;
    const float u = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * t);
    const float p = u * (0.254829592f + u * (-0.284496736f + u * (1.421413741f +
                    u * (-1.453152027f + u * 1.061405429f))));
    const float h = 0.5f * p * __builtin_amdgcn_exp2f(-1.44269504088896341f * t * t);
    return x * (x >= 0.0f ? 1.0f - h : h);
}

// Map a workgroup to (group g, tile_m, tile_n).  Workgroups are dealt
// round-robin to the 8 XCDs (XCD = pid % 8), so each XCD executes its ids
// local = pid / 8 in order.  Every group's tile grid is split into 8
// contiguous ranges, one per XCD, and an XCD walks its range of group 0, then
// of group 1, ...: all XCDs work on the same group (the same weight matrix)
// at the same time and one group's tail overlaps the next group's head.
// Inside a range, tiles walk the output GROUP_M tile-rows at a time.  Returns
// false for the few padding workgroups of XCDs with one tile fewer per group.
__device__ __forceinline__ bool tile_coords(int pid, int groups, int tiles_m, int tiles_n,
                                            int& g, int& tm, int& tn) {
    const int ntiles = tiles_m * tiles_n;
    const int xcd = pid & 7, local = pid >> 3;
    const int per = ntiles >> 3, rem = ntiles & 7;
    const int cnt = per + (xcd < rem ? 1 : 0);         // this XCD's tiles per group
    if (cnt == 0) return false;
    g = local / cnt;
    if (g >= groups) return false;
    const int id = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local % cnt;
    const int width = GROUP_M * tiles_n;
    const int group = id / width;
    const int first_m = group * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_group = id - group * width;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
    return true;
}

// The order used when every group shares its A operand (the activations X
// of the column-parallel products of all ranks): XCD x owns tile-rows
// [x*band, (x+1)*band) of every group and walks them GROUP_M rows at a time;
// for each such row block it visits all groups' column tiles before moving
// on, so the row block of the shared X stays resident in the last-level
// cache while the groups' weights stream past.  Needs tiles_m % 8 == 0.
__device__ __forceinline__ bool tile_coords_band(int pid, int groups, int tiles_m, int tiles_n,
                                                 int& g, int& tm, int& tn) {
    const int xcd = pid & 7, local = pid >> 3;
    const int band = tiles_m >> 3;
    const int per_block = GROUP_M * tiles_n;           // one row block of one group
    const int rb = local / (groups * per_block);
    const int rest = local - rb * (groups * per_block);
    g = rest / per_block;
    const int in_block = rest - g * per_block;
    const int first = rb * GROUP_M;
    if (first >= band) return false;
    const int gsize = min(band - first, GROUP_M);
    if (in_block >= gsize * tiles_n) return false;
    tm = xcd * band + first + in_block % gsize;
    tn = in_block / gsize;
    return true;
}

template <bool OUT_BF16, bool GELU, bool CHECK_K>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(
    GemmBatch batch, int64_t lda, int64_t ldb, int64_t ldc,
    int M, int N, int K, int tiles_m, int tiles_n)
{
    // Two stages as two separate LDS objects: every access below names its
    // stage statically, which lets the compiler see that reads of one stage
    // do not depend on the direct-to-LDS loads still landing in the other.
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];

    int grp, tm, tn;
    if (batch.band ? !tile_coords_band(blockIdx.x, batch.count, tiles_m, tiles_n, grp, tm, tn)
                   : !tile_coords(blockIdx.x, batch.count, tiles_m, tiles_n, grp, tm, tn))
        return;
    const int m0 = tm * BM, n0 = tn * BN;
    const __bf16* __restrict__ A = batch.A[grp];
    const __bf16* __restrict__ B = batch.B[grp];
    const float* __restrict__ bias = batch.bias[grp];
    void* __restrict__ C = batch.C[grp];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = (wid & 3) >> 1, wn = wid & 1, wh = wid >> 2;

    const __bf16* a_tile = A + (int64_t)m0 * lda;
    const __bf16* b_tile = B + n0;

    // ---- global -> LDS: direct (DMA) 16-byte buffer loads ---------------------
    // A buffer_load_dwordx4 ... lds instruction writes 64 lanes x 16 B = 1 KiB
    // contiguously in LDS (lane l at M0 + 16 l), so the swizzled LDS layout is
    // produced by choosing which global unit each lane fetches.  Wave w fills
    // 4 KiB of each operand tile with 4 instructions each:
    //   A: instruction j, lane l -> row 32w + 8j + l/8 (128 B rows), physical unit l%8
    //   B: instruction j, lane l -> K row 8w + 2j + l/32 (512 B rows), physical unit l%32
    // and the logical unit is the physical one XOR the row's swizzle.
    unsigned a_off[LOADS], b_off[LOADS];
    int a_kcol[LOADS], b_krow[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int r = 32 * wid + 8 * j + (lane >> 3);
        const int u = (lane & 7) ^ ((r >> 1) & 7);
        a_kcol[j] = u * 8;
        a_off[j] = (m0 + r) < M ? (unsigned)(r * lda + u * 8) * 2u : OOB;
        const int kr = 8 * wid + 2 * j + (lane >> 5);
        const int ub = (lane & 31) ^ ((kr & 3) << 2);
        b_krow[j] = kr;
        b_off[j] = (n0 + ub * 8) < N ? (unsigned)(kr * ldb + ub * 8) * 2u : OOB;
    }
    auto dma_tile = [&](int k0, char* stage) {
        // a tile past the last one gets an empty range: all loads write zeros
        const int nrec = k0 < K ? 0x7ffffff0 : 0;
        const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(a_tile + k0), (short)0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(b_tile + (int64_t)k0 * ldb), (short)0, nrec, 0x00020000);
        char* sa = stage + wid * 4096;
        char* sb = stage + A_BYTES + wid * 4096;
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ar, LDS_PTR(void, sa + j * 1024), 16,
                (!CHECK_K || (k0 + a_kcol[j]) < K) ? a_off[j] : OOB, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                br, LDS_PTR(void, sb + j * 1024), 16,
                (!CHECK_K || (k0 + b_krow[j]) < K) ? b_off[j] : OOB, 0, 0, 0);
    };
    const int nk = (K + BK - 1) / BK;

    // ---- LDS -> register operand addresses (MFMA 16x16x32) -------------------
    // A operand: lane holds row (lane & 15), K values 8*(lane >> 4) .. +7 of the
    // 32-wide k-step.
    const int a_r = wm * 128 + (lane & 15);
    const int a_swz = (a_r >> 1) & 7;
    unsigned a_rd[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        a_rd[kk] = a_r * 128 + (((kk * 4 + (lane >> 4)) ^ a_swz) << 4);
    // B operand via transpose reads: the 16-lane group g reads K rows 8g..8g+3
    // (and +4 for the second read) of 16 columns; lane gi addresses row
    // (gi >> 2), columns 4*(gi & 3)..+3 and receives column gi.
    const int g = lane >> 4, gi = lane & 15;
    const int b_row = 8 * g + (gi >> 2);              // + 32*kk (+4 for the second half)
    unsigned b_rd[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const int col = wn * 128 + wh * 64 + nj * 16 + 4 * (gi & 3);
        const int unit = col >> 3;
        b_rd[nj] = A_BYTES + b_row * 512 + ((unit ^ ((b_row & 3) << 2)) << 4) + (col & 7) * 2;
    }

    f32x4 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    bf16x8 fa[NI], fb[2][NJ];
    auto load_b = [&](bf16x8 (&b)[NJ], const char* base, int kk) {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const char* p = base + b_rd[nj] + kk * 32 * 512;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p + 4 * 512));
            b[nj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    auto load_a = [&](int mi, const char* base, int kk) {
        fa[mi] = *(const bf16x8*)(base + a_rd[kk] + mi * 16 * 128);
    };
    // MFMAs of one k-step on fa / bc; the next k-step's operands come from
    // (nbase, nkk): B into bn first, each A block into fa[mi] after its last use
    auto kstep = [&](const bf16x8 (&bc)[NJ], bf16x8 (&bn)[NJ], const char* nbase, int nkk) {
        load_b(bn, nbase, nkk);
#pragma unroll
        for (int mi = 0; mi < NI; ++mi) {
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj)
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], bc[nj], acc[mi][nj], 0, 0, 0);
            load_a(mi, nbase, nkk);
        }
    };

    dma_tile(0, lds0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA has landed
    __syncthreads();
    dma_tile(BK, lds1);
    load_b(fb[0], lds0, 0);
#pragma unroll
    for (int mi = 0; mi < NI; ++mi) load_a(mi, lds0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // one K tile = two 32-wide k-steps; the barrier that publishes the next
    // tile sits before the second, whose operand reloads read the next tile
    auto tile = [&](const char* cur_c, char* cur, const char* nxt, int k_next2) {
        kstep(fb[0], fb[1], cur_c, 1);
        sched_kstep<0>();
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                            // next tile visible; `cur` free
        dma_tile(k_next2, cur);                     // empty range past the last tile
        kstep(fb[1], fb[0], nxt, 0);
        sched_kstep<2 * LOADS>();
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        tile(lds0, lds0, lds1, (kt + 2) * BK);
        tile(lds1, lds1, lds0, (kt + 3) * BK);
    }
    if (kt < nk) tile(lds0, lds0, lds1, (kt + 2) * BK);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // ---- epilogue ------------------------------------------------------------
    // Lane holds column (lane & 15) and rows 4*(lane >> 4) + i of each 16x16
    // block.  Staged rows r and r+4, r+8, r+12 (one store instruction) get
    // their units XOR-ed apart so the LDS writes do not conflict.
    const int lcol = wn * 128 + wh * 64 + (lane & 15);        // + 16*nj
    float bv[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
        bv[nj] = (bias && n0 + lcol + 16 * nj < N) ? bias[n0 + lcol + 16 * nj] : 0.0f;
    auto value = [&](int mi, int nj, int r) {
        const float v = acc[mi][nj][r] + bv[nj];
        return GELU ? gelu(v) : v;
    };
    if constexpr (OUT_BF16) {
        char* half = wm ? lds1 : lds0;
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            const int lc = lcol + 16 * nj;
#pragma unroll
            for (int mi = 0; mi < NI; ++mi)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lr = mi * 16 + 4 * (lane >> 4) + r;
                    *(__bf16*)(half + lr * 512 + (((lc >> 3) ^ (((lr >> 2) & 3) << 1)) << 4) +
                               (lc & 7) * 2) = (__bf16)value(mi, nj, r);
                }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8192 / NTHREADS; ++i) {
            const int idx = i * NTHREADS + tid;
            const int row = idx >> 5, unit = idx & 31, lr = row & 127;
            const char* src = (row < 128 ? lds0 : lds1) + lr * 512 +
                              ((unit ^ (((lr >> 2) & 3) << 1)) << 4);
            const int grow = m0 + row, gcol = n0 + unit * 8;
            if (grow < M && gcol < N)
                *(bf16x8*)((__bf16*)C + (int64_t)grow * ldc + gcol) = *(const bf16x8*)src;
        }
    } else {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            char* half = wm ? lds1 : lds0;
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) {
                const int lc = lcol + 16 * nj;
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = m2 * 16 + 4 * (lane >> 4) + r;
                        *(float*)(half + q * 1024 + (((lc >> 2) ^ (((q >> 2) & 3) << 2)) << 4) +
                                  (lc & 3) * 4) = value(4 * p + m2, nj, r);
                    }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8192 / NTHREADS; ++i) {
                const int idx = i * NTHREADS + tid;
                const int lrow = idx >> 6, unit = idx & 63, q = lrow & 63;
                const char* src = (lrow < 64 ? lds0 : lds1) + q * 1024 +
                                  ((unit ^ (((q >> 2) & 3) << 2)) << 4);
                const int grow = m0 + (lrow >> 6) * 128 + 64 * p + q, gcol = n0 + unit * 4;
                if (grow < M && gcol < N)
                    *(f32x4*)((float*)C + (int64_t)grow * ldc + gcol) = *(const f32x4*)src;
            }
            if (p == 0) __syncthreads();
        }
    }
}

}  // namespace

hipError_t gemm_bf16_batched(const GemmBatch& batch, int64_t lda, int64_t ldb, int64_t ldc,
                             int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                             hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    GemmBatch b = batch;
    bool shared_a = b.count > 1;
    for (int i = 1; i < b.count; ++i) shared_a = shared_a && b.A[i] == b.A[0];
    b.band = (shared_a && tiles_m % 8 == 0) ? 1 : 0;
    const int per_xcd = b.band ? ((tiles_m / 8 + GROUP_M - 1) / GROUP_M) * GROUP_M * tiles_n
                               : (tiles_m * tiles_n + 7) / 8;
    const dim3 grid(8 * per_xcd * b.count), block(NTHREADS);
    const bool ck = (K % BK) != 0;
#define TP_GEMM(OB, GL, CK) hipLaunchKernelGGL((gemm_bf16_kernel<OB, GL, CK>), grid, block, 0, \
        stream, b, lda, ldb, ldc, (int)M, (int)N, (int)K, tiles_m, tiles_n)
    if (out_bf16 && gelu)  { if (ck) TP_GEMM(true, true, true);   else TP_GEMM(true, true, false); }
    else if (out_bf16)     { if (ck) TP_GEMM(true, false, true);  else TP_GEMM(true, false, false); }
    else if (gelu)         { if (ck) TP_GEMM(false, true, true);  else TP_GEMM(false, true, false); }
    else                   { if (ck) TP_GEMM(false, false, true); else TP_GEMM(false, false, false); }
#undef TP_GEMM
    return hipGetLastError();
}

hipError_t gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                     const float* bias, void* C, int64_t ldc,
                     int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                     hipStream_t stream)
{
    GemmBatch b = {};
    b.A[0] = (const __bf16*)A;
    b.B[0] = (const __bf16*)B;
    b.bias[0] = bias;
    b.C[0] = C;
    b.count = 1;
    return gemm_bf16_batched(b, lda, ldb, ldc, M, N, K, out_bf16, gelu, stream);
}

}  // namespace tpk

