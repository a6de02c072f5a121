// bf16 x bf16 -> f32-accumulate GEMM for gfx950 (CDNA4) with fused epilogues.
//
// Computes C[M,N] = epi(op(A)·op(B) + bias[N]).  In the forward layout (NN)
// A [M,K] is row-major with K contiguous (the activations X) and B [K,N] is
// row-major with N contiguous (a weight in the [in, out] layout of the
// Megatron explainer's Y = X @ W).  This is the product behind the
// column-parallel layer (epilogue: + bias, GeLU, store bf16:
// "图解Transformer并行计算" §2.1, Y'_i = GeLU(X·A_i)) and the row-parallel
// layer (epilogue: store the f32 partial, §2.1 Z_i = Y'_i·B_i).  The backward
// of the MLP share (§2.2) also needs B stored [N,K] (NT: dY' = dZ·B_i^T,
// dX_i = dY·A_i^T) and A stored [K,M] (TN: dB_i = Y'^T·dZ, dA_i = X^T·dY).
// An operand tile is staged either K-contiguous (read with 16-byte LDS reads)
// or M/N-contiguous (read with the LDS transpose read), whichever its memory
// layout is; nothing is transposed in memory.
//
// Epilogues: none; + bias and GeLU; GeLU backward (C = (A·B)·GeLU'(Y) with the
// saved pre-activation Y read as `aux`); the training forward's dual store
// (C = GeLU(A·B + bias) and aux = A·B + bias, both bf16); and the
// cross-entropy statistics of vocab-parallel logits (per row and column tile
// the maximum and the exp-sum, plus the target's logit; no logits stored).
//
// Design: one 256x256 output tile per workgroup of 8 waves (two per SIMD);
// a launch whose 256-column tiles would leave the last wave of workgroups
// mostly empty uses 256x192 tiles instead (8x3 blocks per wave), products at
// most 128 columns wide use 256x128 tiles (8x2 blocks per wave), and the
// large forward and input-gradient products use 256x384 tiles (a kernel of
// their own, gemm_bf16_w384_kernel below: 5/6 of the operand bytes per
// FLOP); the launcher's rule picks the width.  Given spare device memory, a
// launch with f32 output may also split the tiles of its partly filled last
// wave over K (see split_ways).
//  * wave w owns a 128x64 sub-tile: rows 128*((w&3)>>1), columns
//    128*(w&1) + 64*(w>>2); that is 8x4 MFMA 16x16x32 bf16 blocks with 128
//    f32 accumulators per lane.  The two waves on a SIMD (w and w+4) take the
//    two 64-column halves of one 128x128 quadrant, so while one of them waits
//    on memory the other keeps the SIMD's matrix core busy.  (16x16x32 rather
//    than 32x32x16: with two waves per SIMD it sustains ~10% more MFMA
//    throughput on MI355X under the power limit, measured, for the same
//    operand bytes per FLOP);
//  * K advances in 64-wide steps; the A and B tiles of a step (32 KiB each)
//    are staged in LDS, double-buffered (128 KiB of the 160 KiB per CU); the
//    loads of a step go out over the first 20 of the 32 MFMAs of a k-step;
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
//  * epilogue: every output tile is staged through the (then idle) LDS and
//    written with 16-byte row-contiguous stores; all output stores carry the
//    non-temporal hint (they stream past the L2);
//
// Measured on MI355X (rocprofv3 counters, GeLU GEMM at the 175B layer shape,
// 256x256 tiles): the shader clock settles at ~1.7 GHz under the power limit
// and the matrix cores are busy ~77% of it (~81% with 256x384 tiles, whose
// clock then settles ~0.1 GHz lower).  What idles them is mostly the global -> LDS stream:
// without the K loop's loads (a probe that reuses stale tiles) MFMA busy
// reaches ~85% at the same clock.  The texture data path that carries the
// loads is busy ~96% of the time, over half of it waiting on the L2 (~400
// cycles per request on average); more pipeline stages do not help (a
// 4-stage BK=32 version measured the same), and cache-policy bits do not
// either (non-temporal loads halve throughput: they defeat the L2 sharing
// that the tile order sets up).
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "tp_kernels.h"

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int BM = 256, BN = 256, BK = 64;    // BN: the LDS tile's width (a tile may use 192)
constexpr int NWAVES = 8, NTHREADS = NWAVES * 64;
constexpr int A_BYTES = BM * BK * 2;          // 32 KiB
constexpr int B_BYTES = BK * BN * 2;          // 32 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 4;
constexpr unsigned OOB = 0x80000000u;         // any offset >= num_records reads 0
constexpr int NI = 8;                         // 16x16 MFMA blocks per wave along M
// Blocks per wave along N: 4 (a 256-column tile), 3 (192 columns, for
// products whose 256-column tile count leaves the last wave of workgroups
// mostly empty) or 2 (128 columns, for products at most 128 wide, which a
// 256-column tile would leave half idle); see the launcher.
constexpr int NJ_MAX = 4;
constexpr int LOADS = 4;                      // A (and B) loads per wave per K tile

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// MFMAs of a k-step over which its V direct-to-LDS loads are spread.  The
// loads go out early, over the first 20 of the 32 MFMAs (measured on the
// three forward GEMMs of the block at the 175B layer shape: +2% over spreading
// them across all 32; over the first 8, 12 or 16 or the last 16 it was
// slower).
constexpr int DMA_WINDOW = 20;

// One 32-wide k-step of a wave: 8·NJ MFMAs (A block mi = I/NJ against the NJ
// B blocks); the next k-step's B reads (DB LDS instructions per block) go out
// over the first 8 MFMAs and each A block's reload (DA instructions) right
// after its last MFMA; V direct-to-LDS loads are spread evenly over the
// first DMA_WINDOW·NJ/4 MFMAs (the same share of the k-step).
template <int V, int DA, int DB, int NJ, int I>
__device__ __forceinline__ void sched_step() {
    constexpr int window = DMA_WINDOW * NJ / NJ_MAX;
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    constexpr int nb = I < 8 ? ((I + 1) * NJ * DB) / 8 - (I * NJ * DB) / 8 : 0;
    constexpr int nds = nb + (I % NJ == NJ - 1 ? DA : 0);
    if constexpr (nds > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, nds, 0);
    constexpr int nv = I < window ? ((I + 1) * V) / window - (I * V) / window : 0;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, nv, 0);
    if constexpr (I + 1 < NI * NJ) sched_step<V, DA, DB, NJ, I + 1>();
}
template <int V, int DA, int DB, int NJ>
__device__ __forceinline__ void sched_kstep() {
    sched_step<V, DA, DB, NJ, 0>();
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

// GeLU'(x) = Phi(x) + x·phi(x), phi the standard normal density; Phi from the
// same erfc approximation, and phi(x) = exp(-x^2/2)/sqrt(2 pi) shares its exp.
__device__ __forceinline__ float gelu_grad(float x) {
    const float t = fabsf(x) * 0.70710678118654752f;
    const float u = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * t);
    const float p = u * (0.254829592f + u * (-0.284496736f + u * (1.421413741f +
                    u * (-1.453152027f + u * 1.061405429f))));
    const float e = __builtin_amdgcn_exp2f(-1.44269504088896341f * t * t);
    const float h = 0.5f * p * e;
    return (x >= 0.0f ? 1.0f - h : h) + x * e * 0.39894228040143268f;
}

// Map a workgroup to (group g, tile_m, tile_n).  Workgroups are dealt
// round-robin to the 8 XCDs (XCD = pid % 8), so each XCD executes its ids
// local = pid / 8 in order.  Every group's tile grid is split into 8
// contiguous ranges, one per XCD, and an XCD walks its range of group 0, then
// of group 1, ...: all XCDs work on the same group (the same weight matrix)
// at the same time and one group's tail overlaps the next group's head.
// Inside a range, tiles walk the output GROUP_M tile-rows at a time.  Returns
// false for the few padding workgroups of XCDs with fewer tiles.
__device__ __forceinline__ bool tile_coords(int pid, const GemmBatch& b, int bn, int& g, int& tm,
                                            int& tn) {
    const int xcd = pid & 7;
    int local = pid >> 3;
    for (g = 0; g < b.count; ++g) {
        const int tiles_m = (b.M[g] + BM - 1) / BM, tiles_n = (b.N[g] + bn - 1) / bn;
        const int ntiles = tiles_m * tiles_n;
        const int per = ntiles >> 3, rem = ntiles & 7;
        const int cnt = per + (xcd < rem ? 1 : 0);          // this XCD's tiles of group g
        if (local < cnt) {
            const int id = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) +
                           local;
            const int width = GROUP_M * tiles_n;
            const int group = id / width;
            const int first_m = group * GROUP_M;
            const int gsize = min(tiles_m - first_m, GROUP_M);
            const int in_group = id - group * width;
            tm = first_m + in_group % gsize;
            tn = in_group / gsize;
            return true;
        }
        local -= cnt;
    }
    return false;
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

// Swizzle of an M/N-contiguous tile (64 K rows of 32 16-byte units): logical
// unit u of K row r sits at physical unit u ^ mc_swz(r).  A transpose read
// has each 16-lane group g read 32 contiguous bytes (two units) of the four
// rows 8g..8g+3; the XOR spreads the eight rows that two neighbouring groups
// read (r & 3 and r & 8 differ) over eight distinct 32-byte bank windows,
// while keeping a row's two units adjacent.
__device__ __forceinline__ int mc_swz(int r) { return ((r & 3) << 2) | (((r >> 3) & 1) << 1); }

// K position, relative to the tile's k0, of the unit that lane fetches with
// direct-to-LDS load j of a K-contiguous tile (row 32w + 8j + lane/8, logical
// unit (lane % 8) ^ ((row >> 1) & 7)).  Only the K-tail variant tests it, and
// recomputes it there rather than holding it in registers.
__device__ __forceinline__ int kc_kpos(int lane, int j) {
    return ((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) * 8;
}

// Output tiles are stored with the non-temporal hint: this launch does not
// read them again, and streaming them past the L2 keeps resident the operand
// lines that concurrently running tiles share (measured: +3.4% on the GeLU
// GEMM, +3.3% on the f32-output W_o GEMM, +2% on the row GEMM; the TN weight
// gradients are unchanged within noise).
template <typename T>
__device__ __forceinline__ void st_out(T v, T* p) { __builtin_nontemporal_store(v, p); }

// Cross-entropy statistics of one 128-column piece of a logits row, held by
// 32 lanes (lanes 0..31 or 32..63 of the wave; lane's 4 columns from gcol): the
// maximum m over the columns below N and sum_j exp(logit_j - m), reduced over
// the 32 lanes in a fixed order; the half's first lane writes (m, sum) at
// out + 2·(lane >> 5).  Both output-tile widths build their statistics from
// these pieces, so the statistics do not depend on the width.
__device__ __forceinline__ void ce_half_stats(const f32x4& v, int gcol, int N, int lane, float* out) {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, gcol + e < N ? v[e] : -INFINITY);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sm = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        sm += gcol + e < N ? __builtin_amdgcn_exp2f((v[e] - mx) * 1.44269504088896341f) : 0.0f;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) sm += __shfl_xor(sm, o);
    // a piece that starts at or past N has no columns and is not written
    if ((lane & 31) == 0 && gcol < N) *(float2*)(out + 2 * (lane >> 5)) = make_float2(mx, sm);
}

template <int LAYOUT, int EPI, bool OUT_BF16, bool CHECK_K, int NJ>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(
    GemmBatch batch, int64_t ldaux, int K)
{
    constexpr bool A_MC = LAYOUT == GEMM_TN;    // A stored [K,M]: M contiguous
    constexpr bool B_KC = LAYOUT == GEMM_NT;    // B stored [N,K]: K contiguous
    // Output tile BM x TN.  With NJ = 3 (2) the tile is 192 (128) columns
    // wide: the LDS layout stays 256 wide and its last 64 (128) columns are
    // loaded as zeros (their lanes get out-of-range offsets) and never read.
    constexpr int TN = 64 * NJ;
    static_assert(NJ >= 2 && NJ <= NJ_MAX, "128-, 192- or 256-column tiles");
    static_assert(EPI != EPI_CE_STATS || NJ == NJ_MAX, "the statistics use 256-column tiles");
    // Two stages as two separate LDS objects: every access below names its
    // stage statically, which lets the compiler see that reads of one stage
    // do not depend on the direct-to-LDS loads still landing in the other.
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_BYTES];

    // With a split last wave (f32 output, no epilogue, whole K steps) the
    // tail workgroups id = split_from + part·split_tail + j all take tile
    // split_from + j, part `part` of its K range; the id stays congruent to
    // the tile's own modulo 8 when split_tail is a multiple of 8 (the CU
    // count is), so the tile keeps its XCD.
    constexpr bool SPLITS = EPI == EPI_NONE && !OUT_BF16 && !CHECK_K;
    int pid = blockIdx.x, part = 0;
    const bool split_wg = SPLITS && batch.split_ways > 1 && pid >= batch.split_from;
    if (split_wg) {
        const int j = pid - batch.split_from;
        part = j / batch.split_tail;
        pid = batch.split_from + j % batch.split_tail;
    }
    int grp, tm, tn;
    if (batch.band ? !tile_coords_band(pid, batch.count, (batch.M[0] + BM - 1) / BM,
                                       (batch.N[0] + TN - 1) / TN, grp, tm, tn)
                   : !tile_coords(pid, batch, TN, grp, tm, tn))
        return;
    const int M = batch.M[grp], N = batch.N[grp];
    const int64_t lda = batch.lda[grp], ldb = batch.ldb[grp];
    int64_t ldc = batch.ldc[grp];
    const int m0 = tm * BM, n0 = tn * TN;
    const __bf16* __restrict__ A = batch.A[grp];
    const __bf16* __restrict__ B = batch.B[grp];
    const float* __restrict__ bias = batch.bias[grp];
    void* __restrict__ C = batch.C[grp];
    __bf16* aux = batch.aux[grp];
    if (split_wg) {
        const int kr = K / batch.split_ways, k0 = part * kr;
        A += A_MC ? (int64_t)k0 * lda : k0;
        B += B_KC ? k0 : (int64_t)k0 * ldb;
        K = kr;
        if (part > 0) {
            // block (part - 1, j) of the workspace, addressed so that the
            // epilogue's C + row·ldc + col lands on the tile's element
            // (row - m0, col - n0) of that block
            const int64_t blk = (int64_t)(part - 1) * batch.split_tail + (pid - batch.split_from);
            C = (void*)((uintptr_t)(batch.split_ws + blk * (BM * TN)) -
                        (uintptr_t)(((int64_t)m0 * TN + n0) * 4));
            ldc = TN;
            bias = nullptr;
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = (wid & 3) >> 1, wn = wid & 1, wh = wid >> 2;

    const __bf16* a_tile = A_MC ? A + m0 : A + (int64_t)m0 * lda;
    const __bf16* b_tile = B_KC ? B + (int64_t)n0 * ldb : B + n0;

    // ---- global -> LDS: direct (DMA) 16-byte buffer loads ---------------------
    // A buffer_load_dwordx4 ... lds instruction writes 64 lanes x 16 B = 1 KiB
    // contiguously in LDS (lane l at M0 + 16 l), so the swizzled LDS layout is
    // produced by choosing which global unit each lane fetches.  Wave w fills
    // 4 KiB of each operand tile with 4 instructions, lane l of instruction j:
    //   K-contiguous tile (256 rows x 64 K, 128 B rows): row 32w + 8j + l/8,
    //     physical unit l%8, logical unit = physical ^ ((row >> 1) & 7);
    //   M/N-contiguous tile (64 K rows x 256, 512 B rows): K row 8w + 2j + l/32,
    //     physical unit l%32, logical unit = physical ^ mc_swz(K row).
    // The offsets are loop-invariant; a K step only moves the scalar base.
    unsigned a_off[LOADS], b_off[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int r = 32 * wid + 8 * j + (lane >> 3);
        const int u = (lane & 7) ^ ((r >> 1) & 7);
        const int kr = 8 * wid + 2 * j + (lane >> 5);
        const int ub = (lane & 31) ^ mc_swz(kr);
        if (A_MC)
            a_off[j] = (m0 + ub * 8) < M ? (unsigned)(kr * lda + ub * 8) * 2u : OOB;
        else
            a_off[j] = (m0 + r) < M ? (unsigned)(r * lda + u * 8) * 2u : OOB;
        if (B_KC)
            b_off[j] = (n0 + r) < N && (NJ == NJ_MAX || r < TN) ? (unsigned)(r * ldb + u * 8) * 2u : OOB;
        else
            b_off[j] = (n0 + ub * 8) < N && ub * 8 < TN ? (unsigned)(kr * ldb + ub * 8) * 2u : OOB;
    }
    auto dma_tile = [&](int k0, char* stage) {
        // A tile past the last one gets an empty range: all loads write zeros.
        // In the K-tail variant, an operand stored with K as its row index gets
        // a range ending at row K, so its rows past K read zeros the same way;
        // a K-contiguous operand tests each unit's K position instead.
        const int nrec = k0 < K ? 0x7ffffff0 : 0;
        auto tail = [&](int64_t ld) -> int {      // wave-uniform
            const int64_t bytes = (int64_t)(K - k0) * ld * 2;
            return __builtin_amdgcn_readfirstlane(
                bytes <= 0 ? 0 : (int)(bytes < 0x7ffffff0 ? bytes : 0x7ffffff0));
        };
        const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(A_MC ? a_tile + (int64_t)k0 * lda : a_tile + k0), (short)0,
            (CHECK_K && A_MC) ? tail(lda) : nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(B_KC ? b_tile + k0 : b_tile + (int64_t)k0 * ldb), (short)0,
            (CHECK_K && !B_KC) ? tail(ldb) : nrec, 0x00020000);
        char* sa = stage + wid * 4096;
        char* sb = stage + A_BYTES + wid * 4096;
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ar, LDS_PTR(void, sa + j * 1024), 16,
                (!CHECK_K || A_MC || k0 + kc_kpos(lane, j) < K) ? a_off[j] : OOB, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                br, LDS_PTR(void, sb + j * 1024), 16,
                (!CHECK_K || !B_KC || k0 + kc_kpos(lane, j) < K) ? b_off[j] : OOB, 0, 0, 0);
    };
    // with a lower-triangular A only the K steps up to the tile's last row
    // contribute (causal_k); the loop and the tail handling see a shorter K
    const int nk_all = (K + BK - 1) / BK;
    const int nk = batch.causal_k ? min(nk_all, (m0 + BM + BK - 1) / BK) : nk_all;

    // ---- LDS -> register operand addresses (MFMA 16x16x32) -------------------
    // An MFMA operand block: lane holds row/column (lane & 15) of 16 and the K
    // values 8*(lane >> 4) .. +7 of the 32-wide k-step.
    //  * from a K-contiguous tile: one 16-byte read of row (lane & 15); the
    //    row's swizzle does not depend on which 16-row block is read;
    //  * from an M/N-contiguous tile: two transpose reads; the 16-lane group g
    //    reads K rows 8g..8g+3 (and +4) of 16 columns, lane gi addressing row
    //    (gi >> 2), columns 4*(gi & 3)..+3 and receiving column gi.
    const int g = lane >> 4, gi = lane & 15;
    const unsigned kc_rd = (lane & 15) * 128 + (((lane >> 4) ^ (((lane & 15) >> 1) & 7)) << 4);
    auto mc_rd = [&](int col) -> unsigned {      // col: first column of the block
        const int row = 8 * g + (gi >> 2);
        const int c = col + 4 * (gi & 3);
        return row * 512 + (((c >> 3) ^ mc_swz(row)) << 4) + (c & 7) * 2;
    };
    // For an M-contiguous A, block mi's address is block 0's with bits 5-7
    // XOR-ed by mi (the 16-column blocks differ only in the swizzled unit
    // bits 1-3).
    const unsigned a_rd0 = A_MC ? mc_rd(wm * 128) : wm * 128 * 128 + kc_rd;
    // wave columns: wn·32·NJ + wh·16·NJ (+ 16·nj), i.e. wn·128 + wh·64 for 256-column tiles
    const int wcol = wn * 32 * NJ + wh * 16 * NJ;
    unsigned b_rd[B_KC ? 1 : NJ];
    if constexpr (B_KC) {
        b_rd[0] = A_BYTES + wcol * 128 + kc_rd;
    } else {
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) b_rd[nj] = A_BYTES + mc_rd(wcol + 16 * nj);
    }
    auto read_kc = [&](const char* base, unsigned addr, int blk, int kk) -> bf16x8 {
        // 16-byte unit (4kk + lane>>4) of the row: XOR with kk*4 keeps the swizzle
        return *(const bf16x8*)(base + ((addr + blk * 16 * 128) ^ (kk << 6)));
    };
    auto read_mc = [&](const char* base, unsigned addr, int kk) -> bf16x8 {
        const char* p = base + addr + kk * 32 * 512;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p + 4 * 512));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

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
        for (int nj = 0; nj < NJ; ++nj)
            if constexpr (B_KC) b[nj] = read_kc(base, b_rd[0], nj, kk);
            else b[nj] = read_mc(base, b_rd[nj], kk);
    };
    auto load_a = [&](int mi, const char* base, int kk) {
        if constexpr (A_MC) fa[mi] = read_mc(base, a_rd0 ^ (mi << 5), kk);
        else fa[mi] = read_kc(base, a_rd0, mi, kk);
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
        sched_kstep<0, A_MC ? 2 : 1, B_KC ? 1 : 2, NJ>();
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();                            // next tile visible; `cur` free
        dma_tile(k_next2, cur);                     // empty range past the last tile
        kstep(fb[1], fb[0], nxt, 0);
        sched_kstep<2 * LOADS, A_MC ? 2 : 1, B_KC ? 1 : 2, NJ>();
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
    const int lcol = wcol + (lane & 15);                     // + 16*nj
    float bv[NJ];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj)
        bv[nj] = (bias && n0 + lcol + 16 * nj < N) ? bias[n0 + lcol + 16 * nj] : 0.0f;
    auto value = [&](int mi, int nj, int r) {
        const float v = acc[mi][nj][r] + bv[nj];
        return EPI == EPI_GELU ? gelu(v) : v;
    };
    if constexpr (OUT_BF16 && (EPI == EPI_NONE || EPI == EPI_GELU)) {
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
            if (grow < M && gcol < N && unit * 8 < TN)
                st_out(*(const bf16x8*)src, (bf16x8*)((__bf16*)C + (int64_t)grow * ldc + gcol));
        }
    } else {
        // f32 staging in two passes of 64 rows per half; the store phase writes
        // 1 KiB of one row per store instruction and applies the element-wise
        // epilogues that need a second operand or output.  (Storing a plain
        // f32 tile straight from the accumulators, four 64-byte row segments
        // per instruction, wrote at ~3.1 TB/s against ~5.6 TB/s staged, at
        // K = 64 where the writes bound the launch: staging is +3.9% on the
        // W_o product, K = 1536, and +1.1% on the row product, K = 6144.)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // GeLU backward: the pass's saved pre-activations are loaded before
            // its staging, so that their latency overlaps it instead of
            // stalling the store loop; units past M or N get an offset beyond
            // the buffer range (zeros).  With bf16 output a lane takes two
            // adjacent staged units per step (8 outputs, one 16-byte store;
            // 8-byte stores made the launch ~6% slower), with f32 output one.
            [[maybe_unused]] bf16x4 ypre[8192 / NTHREADS];
            [[maybe_unused]] bf16x8 ypre8[4096 / NTHREADS];
            if constexpr (EPI == EPI_GELU_BWD) {
                const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                    aux + (int64_t)m0 * ldaux + n0, (short)0, 0x7ffffff0, 0x00020000);
                if constexpr (OUT_BF16) {
#pragma unroll
                    for (int i = 0; i < 4096 / NTHREADS; ++i) {
                        const int idx = i * NTHREADS + tid;
                        const int lrow = idx >> 5, u2 = idx & 31, q = lrow & 63;
                        const int r = (lrow >> 6) * 128 + 64 * p + q, c = u2 * 8;
                        const unsigned off = (m0 + r < M && n0 + c < N)
                                                 ? (unsigned)(((int64_t)r * ldaux + c) * 2) : OOB;
                        ypre8[i] = __builtin_bit_cast(
                            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, 0));
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8192 / NTHREADS; ++i) {
                        const int idx = i * NTHREADS + tid;
                        const int lrow = idx >> 6, unit = idx & 63, q = lrow & 63;
                        const int r = (lrow >> 6) * 128 + 64 * p + q, c = unit * 4;
                        const unsigned off = (m0 + r < M && n0 + c < N)
                                                 ? (unsigned)(((int64_t)r * ldaux + c) * 2) : OOB;
                        ypre[i] = __builtin_bit_cast(
                            bf16x4, __builtin_amdgcn_raw_buffer_load_b64(yr, off, 0, 0));
                    }
                }
            }
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
            if constexpr (EPI == EPI_CE_STATS) {
                // one wave holds one whole row of the tile per iteration (its
                // 64 lanes the row's 64 units); each 32-lane half reduces its
                // 128 columns (ce_half_stats) and the target's logit is kept
                const int nsub = (N + 127) / 128;
#pragma unroll 2
                for (int i = 0; i < 8192 / NTHREADS; ++i) {
                    const int lrow = i * (NTHREADS / 64) + wid, q = lrow & 63;
                    const int grow = m0 + (lrow >> 6) * 128 + 64 * p + q, gcol = n0 + lane * 4;
                    if (grow >= M) continue;                // wave-uniform
                    const f32x4 v = *(const f32x4*)((lrow < 64 ? lds0 : lds1) + q * 1024 +
                                                     ((lane ^ (((q >> 2) & 3) << 2)) << 4));
                    ce_half_stats(v, gcol, N, lane, (float*)C + ((int64_t)grow * nsub + 2 * tn) * 2);
                    const int tl = batch.targets[grow] - batch.vstart[grp] - gcol;
                    if (tl >= 0 && tl < 4 && gcol + tl < N) ((float*)aux)[grow] = v[tl];
                }
                if (p == 0) __syncthreads();
                continue;
            }
            if constexpr (OUT_BF16) {
                // GeLU backward or the dual store with bf16 output: lane takes
                // the staged units 2·u2 and 2·u2 + 1 of a row (the XOR keeps
                // them adjacent), 8 outputs per 16-byte store
#pragma unroll
                for (int i = 0; i < 4096 / NTHREADS; ++i) {
                    const int idx = i * NTHREADS + tid;
                    const int lrow = idx >> 5, u2 = idx & 31, q = lrow & 63;
                    const char* rowp = (lrow < 64 ? lds0 : lds1) + q * 1024;
                    const int sw = ((q >> 2) & 3) << 2;
                    const f32x4 v0 = *(const f32x4*)(rowp + (((2 * u2) ^ sw) << 4));
                    const f32x4 v1 = *(const f32x4*)(rowp + (((2 * u2 + 1) ^ sw) << 4));
                    const int grow = m0 + (lrow >> 6) * 128 + 64 * p + q, gcol = n0 + u2 * 8;
                    if (grow < M && gcol < N && u2 * 8 < TN) {
                        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                        const int64_t o = (int64_t)grow * ldc + gcol;
                        if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] *= gelu_grad((float)ypre8[i][e]);
                        }
                        if constexpr (EPI == EPI_DUAL) {
                            bf16x8 y, yp;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                y[e] = (__bf16)v[e];
                                yp[e] = (__bf16)gelu(v[e]);
                            }
                            st_out(y, (bf16x8*)(aux + (int64_t)grow * ldaux + gcol));
                            st_out(yp, (bf16x8*)((__bf16*)C + o));
                        } else {
                            bf16x8 c;
#pragma unroll
                            for (int e = 0; e < 8; ++e) c[e] = (__bf16)v[e];
                            st_out(c, (bf16x8*)((__bf16*)C + o));
                        }
                    }
                }
                if (p == 0) __syncthreads();
                continue;
            }
#pragma unroll
            for (int i = 0; i < 8192 / NTHREADS; ++i) {
                const int idx = i * NTHREADS + tid;
                const int lrow = idx >> 6, unit = idx & 63, q = lrow & 63;
                const char* src = (lrow < 64 ? lds0 : lds1) + q * 1024 +
                                  ((unit ^ (((q >> 2) & 3) << 2)) << 4);
                const int grow = m0 + (lrow >> 6) * 128 + 64 * p + q, gcol = n0 + unit * 4;
                if (grow < M && gcol < N && unit * 4 < TN) {
                    f32x4 v = *(const f32x4*)src;
                    const int64_t o = (int64_t)grow * ldc + gcol;
                    if constexpr (EPI == EPI_GELU_BWD) {
                        const bf16x4 y = ypre[i];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= gelu_grad((float)y[e]);
                    }
                    st_out(v, (f32x4*)((float*)C + o));
                }
            }
            if (p == 0) __syncthreads();
        }
    }
}

// ---- 256 x 384 output tiles ------------------------------------------------
// The K loop of the 256 x 256 kernel is bound by the L2 requests of its
// operand panels, so a wider tile, which needs fewer operand bytes per FLOP
// ((256 + 384) / (256·384) against (256 + 256) / (256·256): 5/6), runs the
// large products faster: measured at the 175B layer shape, grouped over 8
// ranks, 4-5% on the GeLU and QKV products, 6% on the row product and 7% on
// W_o; one rank's input gradients (B stored [N,K]) 6-7%, with results
// bit-identical to the 256-column kernel (each output sees the same MFMA
// sequence over K).
//  * eight waves, wave w owning 128 x 96: rows 128·((w&3)>>1), columns
//    192·(w&1) + 96·(w>>2), i.e. 8 x 6 MFMA 16x16x32 blocks with 192 f32
//    accumulators per lane.  Two waves per SIMD give a wave 256 VGPRs, so the
//    operands are held lean: the six B blocks of the k-step (24 VGPRs) and two
//    A blocks (8).  Row mi's MFMAs run while the A block of row mi+1 is read;
//    in the last row each B block is re-read for the next k-step right after
//    its MFMA;
//  * two 80 KiB stages (A 32 KiB, B 48 KiB) fill the 160 KiB of LDS.  The
//    operand tiles are staged and read as in the 256-column kernel, in the
//    layout their memory has: a K-contiguous tile as rows of 128 bytes read
//    with 16-byte reads, an M/N-contiguous one as 64 K rows (512 bytes for A,
//    768 for B) read with transpose reads, both with the same XOR swizzles
//    (the M/N-contiguous one depends on K row bits 0, 1 and 3 only and keeps a
//    unit inside its aligned group of 16);
//  * the loads of the next K tile go out over the first 30 of the 48 MFMAs of
//    a tile's first k-step (a window of 20 was 1-2% slower, 40 the same); the
//    barrier that publishes them sits before the last row of the second
//    k-step, after the last reads of the current stage;
//  * the output tile is staged through the LDS in two (bf16 values) or four
//    (f32 values) passes in which all eight waves take part; the epilogues
//    that need a second operand or output (GeLU backward, the dual store)
//    work from the f32 stage like the 256-column kernel's.
// K must be a multiple of 64 and there is no causal K bound; the launcher
// picks this kernel by the cost model of gemm_tile_cols().
constexpr int W_NJ = 6, W_TN = 64 * W_NJ;              // 384 columns
constexpr int W_ROWB = W_TN * 2;                        // 768 B per K row of an N-contiguous B tile
constexpr int W_B_BYTES = BK * W_ROWB;                  // 48 KiB
constexpr int W_STAGE = A_BYTES + W_B_BYTES;            // 80 KiB
constexpr int W_BLOADS = W_B_BYTES / (NTHREADS * 16);   // B loads per wave per K tile
constexpr int W_WINDOW = 30;
static_assert(W_BLOADS == 6 && 2 * W_STAGE <= 160 * 1024, "two 80 KiB stages");
template <int V>
using IC = std::integral_constant<int, V>;

// Schedule of one 32-wide k-step, MFMAs I .. R1·6-1 (row mi = I / 6): the A
// read of the next row (DA LDS instructions) after each row's first MFMA, the
// B re-reads (DB instructions each) after the last row's MFMAs, and V
// direct-to-LDS loads spread over the first W_WINDOW MFMAs.
template <int V, int DA, int DB, int I, int R1>
__device__ __forceinline__ void w_sched() {
    constexpr int mi = I / W_NJ, nj = I % W_NJ;
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    constexpr int nds = (nj == 0 ? DA : 0) + (mi == NI - 1 ? DB : 0);
    if constexpr (nds > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, nds, 0);
    constexpr int nv = I < W_WINDOW ? ((I + 1) * V) / W_WINDOW - (I * V) / W_WINDOW : 0;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, nv, 0);
    if constexpr (I + 1 < R1 * W_NJ) w_sched<V, DA, DB, I + 1, R1>();
}

template <int LAYOUT, int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_w384_kernel(GemmBatch batch,
                                                                     int64_t ldaux, int K)
{
    constexpr bool A_MC = LAYOUT == GEMM_TN;    // A stored [K,M]: M contiguous
    constexpr bool B_KC = LAYOUT == GEMM_NT;    // B stored [N,K]: K contiguous
    static_assert(EPI == EPI_NONE || (LAYOUT == GEMM_NN && (EPI == EPI_GELU || EPI == EPI_DUAL)) ||
                  (LAYOUT == GEMM_NT && (EPI == EPI_GELU_BWD || EPI == EPI_CE_STATS)), "epilogue");
    static_assert(EPI != EPI_CE_STATS || !OUT_BF16, "the statistics are f32");
    static_assert(EPI != EPI_DUAL || OUT_BF16, "the dual store is bf16");
    constexpr int DA = A_MC ? 2 : 1, DB = B_KC ? 1 : 2;     // LDS reads per operand block
    __shared__ __attribute__((aligned(1024))) char lds0[W_STAGE];
    __shared__ __attribute__((aligned(1024))) char lds1[W_STAGE];

    int grp, tm, tn;
    if (batch.band ? !tile_coords_band(blockIdx.x, batch.count, (batch.M[0] + BM - 1) / BM,
                                       (batch.N[0] + W_TN - 1) / W_TN, grp, tm, tn)
                   : !tile_coords(blockIdx.x, batch, W_TN, grp, tm, tn))
        return;
    const int M = batch.M[grp], N = batch.N[grp];
    const int64_t lda = batch.lda[grp], ldb = batch.ldb[grp], ldc = batch.ldc[grp];
    const int m0 = tm * BM, n0 = tn * W_TN;
    const __bf16* __restrict__ A = batch.A[grp];
    const __bf16* __restrict__ B = batch.B[grp];
    const float* __restrict__ bias = batch.bias[grp];
    void* __restrict__ C = batch.C[grp];
    __bf16* aux = batch.aux[grp];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = (wid & 3) >> 1, wn = wid & 1, wh = wid >> 2;
    const __bf16* a_tile = A_MC ? A + m0 : A + (int64_t)m0 * lda;
    const __bf16* b_tile = B_KC ? B + (int64_t)n0 * ldb : B + n0;

    // direct-to-LDS loads; rows or columns past M or N get an offset beyond
    // the buffer's range and read zeros.
    //  A, K-contiguous (256 rows of 128 B): load j of wave w fills rows
    //    32w + 8j .. +7, unit (lane%8) ^ ((row>>1)&7);
    //  A, M-contiguous (64 K rows of 32 units): K row 8w + 2j + lane/32, unit
    //    (lane%32) ^ mc_swz(row);
    //  B, N-contiguous (64 K rows of 48 units): load j of wave w fills the
    //    physical units (6w + j)·64 .. +63 of the tile; physical unit p is K
    //    row p / 48, unit p % 48, and holds logical unit (p % 48) ^ mc_swz(row);
    //  B, K-contiguous (384 rows of 128 B): rows 48w + 8j .. +7.
    unsigned a_off[LOADS], b_off[W_BLOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        if constexpr (A_MC) {
            const int kr = 8 * wid + 2 * j + (lane >> 5);
            const int ub = (lane & 31) ^ mc_swz(kr);
            a_off[j] = (m0 + ub * 8) < M ? (unsigned)(kr * lda + ub * 8) * 2u : OOB;
        } else {
            const int r = 32 * wid + 8 * j + (lane >> 3);
            const int u = (lane & 7) ^ ((r >> 1) & 7);
            a_off[j] = (m0 + r) < M ? (unsigned)(r * lda + u * 8) * 2u : OOB;
        }
    }
#pragma unroll
    for (int j = 0; j < W_BLOADS; ++j) {
        if constexpr (B_KC) {
            const int r = 48 * wid + 8 * j + (lane >> 3);
            const int u = (lane & 7) ^ ((r >> 1) & 7);
            b_off[j] = (n0 + r) < N ? (unsigned)(r * ldb + u * 8) * 2u : OOB;
        } else {
            const int p = (W_BLOADS * wid + j) * 64 + lane;
            const int r = p / 48, u = (p % 48) ^ mc_swz(r);
            b_off[j] = (n0 + u * 8) < N ? (unsigned)(r * ldb + u * 8) * 2u : OOB;
        }
    }
    auto dma_tile = [&](int k0, char* stage) __attribute__((always_inline)) {
        const int nrec = k0 < K ? 0x7ffffff0 : 0;     // past the last K tile: zeros
        const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(A_MC ? a_tile + (int64_t)k0 * lda : a_tile + k0), (short)0, nrec,
            0x00020000);
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<__bf16*>(B_KC ? b_tile + k0 : b_tile + (int64_t)k0 * ldb), (short)0, nrec,
            0x00020000);
        char* sa = stage + wid * 4096;
        char* sb = stage + A_BYTES + wid * (W_BLOADS * 1024);
#pragma unroll
        for (int j = 0; j < LOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, LDS_PTR(void, sa + j * 1024), 16,
                                                     a_off[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < W_BLOADS; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(br, LDS_PTR(void, sb + j * 1024), 16,
                                                     b_off[j], 0, 0, 0);
    };
    const int nk = K / BK;

    // operand reads, as in the 256-column kernel: 16-byte reads of a
    // K-contiguous tile, transpose reads of an M/N-contiguous one (rows of
    // 512 bytes for A, 768 for B)
    const int g = lane >> 4, gi = lane & 15;
    const unsigned kc_rd = (lane & 15) * 128 + (((lane >> 4) ^ (((lane & 15) >> 1) & 7)) << 4);
    auto mc_rd = [&](int col, int rowb) -> unsigned {      // col: first column of the block
        const int row = 8 * g + (gi >> 2);
        const int c = col + 4 * (gi & 3);
        return row * rowb + (((c >> 3) ^ mc_swz(row)) << 4) + (c & 7) * 2;
    };
    const unsigned a_rd0 = A_MC ? mc_rd(wm * 128, 512) : wm * 128 * 128 + kc_rd;
    const int wcol = wn * 192 + wh * 96;
    unsigned b_rd[B_KC ? 1 : W_NJ];
    if constexpr (B_KC) {
        b_rd[0] = A_BYTES + wcol * 128 + kc_rd;
    } else {
#pragma unroll
        for (int nj = 0; nj < W_NJ; ++nj) b_rd[nj] = A_BYTES + mc_rd(wcol + 16 * nj, W_ROWB);
    }
    auto tr_read = [&](const char* p, int rowb) __attribute__((always_inline)) -> bf16x8 {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, p + 4 * rowb));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x4 acc[NI][W_NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < W_NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    bf16x8 fa[2], fb[W_NJ];
    auto ld_a = [&](int slot, const char* base, int mi, int kk) __attribute__((always_inline)) {
        // an M-contiguous block mi is block 0's address with bits 5-7 XOR-ed
        // by mi (the 16-column blocks differ only in the swizzled unit bits 1-3)
        if constexpr (A_MC) fa[slot] = tr_read(base + (a_rd0 ^ (mi << 5)) + kk * 32 * 512, 512);
        else fa[slot] = *(const bf16x8*)(base + ((a_rd0 + mi * 16 * 128) ^ (kk << 6)));
    };
    auto ld_b = [&](int nj, const char* base, int kk) __attribute__((always_inline)) {
        if constexpr (B_KC) fb[nj] = *(const bf16x8*)(base + ((b_rd[0] + nj * 16 * 128) ^ (kk << 6)));
        else fb[nj] = tr_read(base + b_rd[nj] + kk * 32 * W_ROWB, W_ROWB);
    };
    // rows [R0, R1) of a 32-wide k-step whose operands come from (cb, ckk);
    // the next k-step's come from (nb, nkk).  The row bounds are compile-time
    // constants so that every accumulator index is one.
    auto rows = [&](auto R0, auto R1, const char* cb, int ckk, const char* nb, int nkk)
                    __attribute__((always_inline)) {
        constexpr int r0 = decltype(R0)::value, r1 = decltype(R1)::value;
#pragma unroll
        for (int mi = r0; mi < r1; ++mi) {
            if (mi < NI - 1) ld_a((mi + 1) & 1, cb, mi + 1, ckk);
            else ld_a(0, nb, 0, nkk);
#pragma unroll
            for (int nj = 0; nj < W_NJ; ++nj) {
                acc[mi][nj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi & 1], fb[nj],
                                                                      acc[mi][nj], 0, 0, 0);
                if (mi == NI - 1) ld_b(nj, nb, nkk);
            }
        }
    };
    // One K tile in stage `cur`.  Its first k-step issues the loads of the
    // next K tile into `oth`, whose last reads came before the previous
    // tile's barrier; the barrier before this tile's last row publishes them.
    auto tile = [&](const char* cur, char* oth, int k_next) __attribute__((always_inline)) {
        dma_tile(k_next, oth);
        rows(IC<0>{}, IC<NI>{}, cur, 0, cur, 1);
        w_sched<LOADS + W_BLOADS, DA, DB, 0, NI>();
        __builtin_amdgcn_sched_barrier(0);
        rows(IC<0>{}, IC<NI - 1>{}, cur, 1, cur, 1);
        w_sched<0, DA, DB, 0, NI - 1>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): this wave's loads have landed
        __syncthreads();                           // `oth` complete; `cur` no longer read
        rows(IC<NI - 1>{}, IC<NI>{}, cur, 1, oth, 0);
        w_sched<0, DA, DB, (NI - 1) * W_NJ, NI>();
        __builtin_amdgcn_sched_barrier(0);
    };

    dma_tile(0, lds0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#pragma unroll
    for (int nj = 0; nj < W_NJ; ++nj) ld_b(nj, lds0, 0);
    ld_a(0, lds0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        tile(lds0, lds1, (kt + 1) * BK);
        tile(lds1, lds0, (kt + 2) * BK);
    }
    if (kt < nk) tile(lds0, lds1, (kt + 1) * BK);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // ---- epilogue ------------------------------------------------------------
    // Lane holds column (lane & 15) and rows 4·(lane >> 4) + r of each 16x16
    // block.  Each pass stages some row blocks of every wave (the waves with
    // wm = 0 into lds0, wm = 1 into lds1; rows four apart get their units
    // XOR-ed apart), then the workgroup writes the staged rows with 16-byte
    // row-contiguous stores.
    const int lcol = wcol + (lane & 15);                     // + 16·nj
    float bv[W_NJ];
#pragma unroll
    for (int nj = 0; nj < W_NJ; ++nj)
        bv[nj] = (bias && n0 + lcol + 16 * nj < N) ? bias[n0 + lcol + 16 * nj] : 0.0f;
    auto value = [&](int mi, int nj, int r) __attribute__((always_inline)) {
        const float v = acc[mi][nj][r] + bv[nj];
        return EPI == EPI_GELU ? gelu(v) : v;
    };
    char* half = wm ? lds1 : lds0;
    if constexpr (OUT_BF16 && (EPI == EPI_NONE || EPI == EPI_GELU)) {
        // two passes of row blocks 4p .. 4p+3 (64 rows of each 128-row half)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int nj = 0; nj < W_NJ; ++nj) {
                const int lc = lcol + 16 * nj;
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = m2 * 16 + 4 * (lane >> 4) + r;
                        *(__bf16*)(half + q * W_ROWB + (((lc >> 3) ^ (((q >> 2) & 3) << 1)) << 4) +
                                   (lc & 7) * 2) = (__bf16)value(4 * p + m2, nj, r);
                    }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 128 * 48 / NTHREADS; ++i) {
                const int idx = i * NTHREADS + tid;
                const int lrow = idx / 48, unit = idx % 48, q = lrow & 63;
                const char* src = (lrow < 64 ? lds0 : lds1) + q * W_ROWB +
                                  ((unit ^ (((q >> 2) & 3) << 1)) << 4);
                const int grow = m0 + (lrow >> 6) * 128 + 64 * p + q, gcol = n0 + unit * 8;
                if (grow < M && gcol < N)
                    st_out(*(const bf16x8*)src, (bf16x8*)((__bf16*)C + (int64_t)grow * ldc + gcol));
            }
            if (p == 0) __syncthreads();
        }
    } else {
        // four passes of row blocks 2p, 2p+1 (32 rows of each half, 1536 B per
        // row).  The store phase applies the element-wise epilogues that need a
        // second operand or output; with bf16 output a lane takes the staged
        // units 2·u2 and 2·u2 + 1 of a row (the XOR keeps them adjacent), 8
        // outputs per 16-byte store.  GeLU backward: the pass's saved
        // pre-activations are loaded right after its staging (whose
        // accumulators are then dead), so that their latency overlaps the
        // barrier; units past M or N read zeros.
        constexpr int UNITS = OUT_BF16 ? 48 : 96;             // per staged row and lane step
        constexpr int PER = 64 * UNITS / NTHREADS;            // store steps per lane per pass
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            [[maybe_unused]] bf16x8 ypre8[OUT_BF16 ? PER : 1];
            [[maybe_unused]] bf16x4 ypre4[OUT_BF16 ? 1 : PER];
#pragma unroll
            for (int nj = 0; nj < W_NJ; ++nj) {
                const int lc = lcol + 16 * nj;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = m2 * 16 + 4 * (lane >> 4) + r;
                        *(float*)(half + q * 1536 + (((lc >> 2) ^ (((q >> 2) & 3) << 2)) << 4) +
                                  (lc & 3) * 4) = value(2 * p + m2, nj, r);
                    }
            }
            if constexpr (EPI == EPI_GELU_BWD) {
                const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                    aux + (int64_t)m0 * ldaux + n0, (short)0, 0x7ffffff0, 0x00020000);
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int idx = i * NTHREADS + tid;
                    const int lrow = idx / UNITS, u = idx % UNITS, q = lrow & 31;
                    const int r = (lrow >> 5) * 128 + 32 * p + q, c = u * (OUT_BF16 ? 8 : 4);
                    const unsigned off = (m0 + r < M && n0 + c < N)
                                             ? (unsigned)(((int64_t)r * ldaux + c) * 2) : OOB;
                    if constexpr (OUT_BF16)
                        ypre8[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, 0));
                    else
                        ypre4[i] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(yr, off, 0, 0));
                }
            }
            __syncthreads();
            if constexpr (EPI == EPI_CE_STATS) {
                // one wave per staged row (64 rows per pass, 8 per wave): all 64
                // lanes take columns 0..255 (4 each), then lanes 0..31 take
                // 256..383 -- three 128-column pieces, each reduced by
                // ce_half_stats as the 256-column kernel does
                const int nsub = (N + 127) / 128;
#pragma unroll 2
                for (int i = 0; i < 64 / NWAVES; ++i) {
                    const int lrow = i * NWAVES + wid, q = lrow & 31;
                    const int grow = m0 + (lrow >> 5) * 128 + 32 * p + q;
                    if (grow >= M) continue;                // wave-uniform
                    const char* rowp = (lrow < 32 ? lds0 : lds1) + q * 1536;
                    const int sw = ((q >> 2) & 3) << 2;
                    float* out = (float*)C + ((int64_t)grow * nsub + 3 * tn) * 2;
                    const int tgt = batch.targets[grow] - batch.vstart[grp];
                    const int gc0 = n0 + lane * 4;
                    const f32x4 v0 = *(const f32x4*)(rowp + ((lane ^ sw) << 4));
                    ce_half_stats(v0, gc0, N, lane, out);
                    if (tgt - gc0 >= 0 && tgt - gc0 < 4 && tgt < N) ((float*)aux)[grow] = v0[tgt - gc0];
                    const int gc1 = n0 + 256 + (lane & 31) * 4;
                    const f32x4 v1 = *(const f32x4*)(rowp + (((64 + (lane & 31)) ^ sw) << 4));
                    // lanes 32..63 see columns past every piece (gcol >= N for
                    // their reduction half, nothing written)
                    ce_half_stats(v1, lane < 32 ? gc1 : N, N, lane, out + 4);
                    if (lane < 32 && tgt - gc1 >= 0 && tgt - gc1 < 4 && tgt < N)
                        ((float*)aux)[grow] = v1[tgt - gc1];
                }
                if (p < 3) __syncthreads();
                continue;
            }
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int idx = i * NTHREADS + tid;
                const int lrow = idx / UNITS, u = idx % UNITS, q = lrow & 31;
                const char* rowp = (lrow < 32 ? lds0 : lds1) + q * 1536;
                const int sw = ((q >> 2) & 3) << 2;
                const int grow = m0 + (lrow >> 5) * 128 + 32 * p + q;
                if constexpr (OUT_BF16) {
                    const int gcol = n0 + u * 8;
                    if (grow < M && gcol < N) {
                        const f32x4 v0 = *(const f32x4*)(rowp + (((2 * u) ^ sw) << 4));
                        const f32x4 v1 = *(const f32x4*)(rowp + (((2 * u + 1) ^ sw) << 4));
                        float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                        const int64_t o = (int64_t)grow * ldc + gcol;
                        if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] *= gelu_grad((float)ypre8[i][e]);
                        }
                        if constexpr (EPI == EPI_DUAL) {
                            bf16x8 y, yp;
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                y[e] = (__bf16)v[e];
                                yp[e] = (__bf16)gelu(v[e]);
                            }
                            st_out(y, (bf16x8*)(aux + (int64_t)grow * ldaux + gcol));
                            st_out(yp, (bf16x8*)((__bf16*)C + o));
                        } else {
                            bf16x8 c;
#pragma unroll
                            for (int e = 0; e < 8; ++e) c[e] = (__bf16)v[e];
                            st_out(c, (bf16x8*)((__bf16*)C + o));
                        }
                    }
                } else {
                    const int gcol = n0 + u * 4;
                    if (grow < M && gcol < N) {
                        f32x4 v = *(const f32x4*)(rowp + ((u ^ sw) << 4));
                        if constexpr (EPI == EPI_GELU_BWD) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] *= gelu_grad((float)ypre4[i][e]);
                        }
                        st_out(v, (f32x4*)((float*)C + (int64_t)grow * ldc + gcol));
                    }
                }
            }
            if (p < 3) __syncthreads();
        }
    }
}

}  // namespace

// Compute units of the current device (256 on MI355X), for the tile-width
// choice; queried once per device.
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {
// Second launch of a split last wave: C += block p of tail tile j for p = 1,
// 2, ... in that order (range 0 is already in C), one workgroup per 64-row
// quarter of a tile, 16-byte units (every group's N and ldc a multiple of 4,
// C 16-byte aligned: checked by the launcher).
__global__ __launch_bounds__(256) void split_fixup_kernel(GemmBatch batch, int tile_cols) {
    const int j = blockIdx.x >> 2, quarter = blockIdx.x & 3;
    int grp, tm, tn;
    if (!tile_coords(batch.split_from + j, batch, tile_cols, grp, tm, tn)) return;
    const int r0 = 64 * quarter, m0 = tm * BM + r0, n0 = tn * tile_cols;
    const int rows = min(64, batch.M[grp] - m0), cols = min(tile_cols, batch.N[grp] - n0);
    if (rows <= 0) return;
    float* C = (float*)batch.C[grp] + (int64_t)m0 * batch.ldc[grp] + n0;
    const int units = tile_cols / 4;
    const int64_t blk = (int64_t)BM * tile_cols;
    const float* ws = batch.split_ws + (int64_t)j * blk + (int64_t)r0 * tile_cols;
    for (int idx = threadIdx.x; idx < 64 * units; idx += 256) {
        const int r = idx / units, c = 4 * (idx - r * units);
        if (r >= rows || c >= cols) continue;
        f32x4* dst = (f32x4*)(C + (int64_t)r * batch.ldc[grp] + c);
        f32x4 acc = *dst;
        for (int p = 1; p < batch.split_ways; ++p)
            acc += *(const f32x4*)(ws + (int64_t)(p - 1) * batch.split_tail * blk +
                                   (int64_t)r * tile_cols + c);
        *dst = acc;
    }
}

// Workgroups of a launch with tiles tn_w columns wide (one 256 x tn_w tile each).
int64_t tile_count(const GemmBatch& b, int tn_w) {
    int64_t t = 0;
    for (int g = 0; g < b.count; ++g)
        t += (int64_t)((b.M[g] + BM - 1) / BM) * ((b.N[g] + tn_w - 1) / tn_w);
    return t;
}

// Whether a launch can take 256 x 384 tiles: the forward (NN) and input-gradient
// (NT) layouts with every epilogue, K a multiple of 64 and no causal K bound.  The weight-gradient layout (TN: both operands M/N-contiguous, eight
// transpose-read addresses for A) does not fit the register budget.
bool wide_ok(const GemmBatch& b, int layout, int epi, int64_t K) {
    if (layout == GEMM_TN) return false;
    const bool epi_ok = epi == EPI_NONE || (layout == GEMM_NN && (epi == EPI_GELU || epi == EPI_DUAL)) ||
                        (layout == GEMM_NT && (epi == EPI_GELU_BWD || epi == EPI_CE_STATS));
    if (!epi_ok || K % BK != 0 || b.causal_k) return false;
    // a K-contiguous B tile spans 384 rows, addressed with 32-bit byte offsets
    for (int g = 0; layout == GEMM_NT && g < b.count; ++g)
        if (b.ldb[g] * 2 * W_TN >= 0x7fffffff) return false;
    return true;
}

}  // namespace

// Output-tile width of a launch: 128 columns when no product is wider (a
// 256-column tile would do the same number of tiles with half its MFMAs on
// zero columns; not for the cross-entropy statistics), else 256 columns, or
// 192 or 384 where a cost model of the waves of workgroups (one workgroup per
// CU) says so.  The cost of a
// wave, in sixteenths of a wave of 256-column tiles: 14 for 192 columns (the
// K loop is bound by the L2 requests of a tile's A and B panels, 256 + 192
// rows against 256 + 256), 23 for 384 (1.5 times the work, measured 4-7%
// faster per FLOP).  Another width is taken only where it saves more than
// 1/8 of a 256-column wave; ties keep the narrower tile.  Measured on MI355X:
// [8192 x 4096]·[4096 x 3072] (384 tiles of 256 columns, 1.5 waves; 512 of
// 192, 2 waves) and the 175B layer shape's products (48 waves of 256-column
// tiles, 32 of 384).
int gemm_tile_cols(const GemmBatch& b, int layout, int epi, int64_t K) {
    if (tile_count(b, 192) > 0x7fffffff / 16) return 256;     // keep the grid size in range
    if (epi != EPI_CE_STATS) {
        bool narrow = true;
        for (int g = 0; g < b.count; ++g) narrow = narrow && b.N[g] <= 128;
        if (narrow) return 128;
    }
    const int64_t cus = cu_count();
    auto waves = [&](int w) { return (tile_count(b, w) + cus - 1) / cus; };
    int best = 256;
    int64_t cost = 16 * waves(256);
    // (the cross-entropy statistics have no 192-column kernel)
    if (epi != EPI_CE_STATS && 14 * waves(192) < cost - 2) {
        best = 192;
        cost = 14 * waves(192);
    }
    if (wide_ok(b, layout, epi, K) && 23 * waves(384) < cost - 2) best = 384;
    return best;
}

namespace {
// The tile kernel of a launch whose width, grid and split are set.
hipError_t launch_tiles(const GemmBatch& b, int tn_w, dim3 grid, int layout, int epi,
                        int64_t ldaux, int64_t K, bool out_bf16, hipStream_t stream)
{
    const int nj = tn_w / 64;
    const dim3 block(NTHREADS);
    if (tn_w == W_TN) {
#define TP_GEMM_W(L, E, OB)                                                                    \
    do {                                                                                       \
        hipLaunchKernelGGL((gemm_bf16_w384_kernel<L, E, OB>), grid, block, 0, stream, b, ldaux, \
                           (int)K);                                                            \
        return hipGetLastError();                                                              \
    } while (0)
        switch (layout) {
        case GEMM_NN:
            if (epi == EPI_NONE) { if (out_bf16) TP_GEMM_W(GEMM_NN, EPI_NONE, true); TP_GEMM_W(GEMM_NN, EPI_NONE, false); }
            if (epi == EPI_GELU) { if (out_bf16) TP_GEMM_W(GEMM_NN, EPI_GELU, true); TP_GEMM_W(GEMM_NN, EPI_GELU, false); }
            if (epi == EPI_DUAL && out_bf16) TP_GEMM_W(GEMM_NN, EPI_DUAL, true);
            break;
        case GEMM_NT:
            if (epi == EPI_NONE) { if (out_bf16) TP_GEMM_W(GEMM_NT, EPI_NONE, true); TP_GEMM_W(GEMM_NT, EPI_NONE, false); }
            if (epi == EPI_GELU_BWD) { if (out_bf16) TP_GEMM_W(GEMM_NT, EPI_GELU_BWD, true); TP_GEMM_W(GEMM_NT, EPI_GELU_BWD, false); }
            if (epi == EPI_CE_STATS && !out_bf16) TP_GEMM_W(GEMM_NT, EPI_CE_STATS, false);
            break;
        default:
            break;
        }
#undef TP_GEMM_W
        return hipErrorInvalidValue;
    }
    const bool ck = (K % BK) != 0;
#define TP_GEMM_NJ(L, E, OB, NJ)                                                               \
    do {                                                                                       \
        if (ck)                                                                                \
            hipLaunchKernelGGL((gemm_bf16_kernel<L, E, OB, true, NJ>), grid, block, 0, stream, \
                               b, ldaux, (int)K);                                              \
        else                                                                                   \
            hipLaunchKernelGGL((gemm_bf16_kernel<L, E, OB, false, NJ>), grid, block, 0,        \
                               stream, b, ldaux, (int)K);                                      \
        return hipGetLastError();                                                              \
    } while (0)
#define TP_GEMM(L, E, OB)                                                                      \
    do {                                                                                       \
        if (nj == 2) TP_GEMM_NJ(L, E, OB, 2);                                                  \
        if (nj == 3) TP_GEMM_NJ(L, E, OB, 3);                                                  \
        TP_GEMM_NJ(L, E, OB, NJ_MAX);                                                          \
    } while (0)
    switch (layout) {
    case GEMM_NN:
        if (epi == EPI_NONE) { if (out_bf16) TP_GEMM(GEMM_NN, EPI_NONE, true); TP_GEMM(GEMM_NN, EPI_NONE, false); }
        if (epi == EPI_GELU) { if (out_bf16) TP_GEMM(GEMM_NN, EPI_GELU, true); TP_GEMM(GEMM_NN, EPI_GELU, false); }
        if (epi == EPI_DUAL && out_bf16) TP_GEMM(GEMM_NN, EPI_DUAL, true);
        break;
    case GEMM_NT:
        if (epi == EPI_NONE) { if (out_bf16) TP_GEMM(GEMM_NT, EPI_NONE, true); TP_GEMM(GEMM_NT, EPI_NONE, false); }
        if (epi == EPI_GELU_BWD) { if (out_bf16) TP_GEMM(GEMM_NT, EPI_GELU_BWD, true); TP_GEMM(GEMM_NT, EPI_GELU_BWD, false); }
        if (epi == EPI_CE_STATS && !out_bf16) TP_GEMM_NJ(GEMM_NT, EPI_CE_STATS, false, NJ_MAX);
        break;
    case GEMM_TN:
        if (epi == EPI_NONE) { if (out_bf16) TP_GEMM(GEMM_TN, EPI_NONE, true); TP_GEMM(GEMM_TN, EPI_NONE, false); }
        break;
    }
#undef TP_GEMM
#undef TP_GEMM_NJ
    return hipErrorInvalidValue;      // a layout / epilogue pair with no kernel
}

// Ways to split each tile of a launch's last wave over K, 0 for none.  With
// W workgroups on C compute units (one each) the last wave holds
// t = W mod C tiles; when t <= C/2 (C/4) the wave can run as 2t (4t)
// workgroups of half (a quarter of) the K loop, taking half (a quarter of)
// a tile's time, at the price of (ways - 1)·t f32 tile blocks written,
// read back and added to C.  Taken from K = 4096 (8192) on, where the
// saved K loop outweighs that traffic, and only with f32 output and no
// epilogue, whole K steps and a caller-provided workspace that holds the
// blocks.
int split_ways(const GemmBatch& b, int tn_w, int64_t workgroups, int epi, int64_t K,
               bool out_bf16) {
    if (!b.split_ws || epi != EPI_NONE || out_bf16 || tn_w == W_TN || b.band || b.causal_k)
        return 0;
    const int64_t cus = cu_count();
    const int64_t tail = workgroups % cus;
    if (tail == 0) return 0;
    for (int g = 0; g < b.count; ++g)
        if (b.N[g] % 4 || b.ldc[g] % 4 || ((uintptr_t)b.C[g] & 15)) return 0;
    for (int ways = 4; ways >= 2; ways /= 2) {
        if (ways * tail > cus || K % (ways * BK) != 0 || K < 2048 * ways) continue;
        if ((ways - 1) * tail * BM * tn_w * 4 <= b.split_ws_bytes) return ways;
    }
    return 0;
}

hipError_t launch(const GemmBatch& b_in, int layout, int epi, int64_t ldaux, int64_t K,
                  bool out_bf16, hipStream_t stream)
{
    const int tn_w = gemm_tile_cols(b_in, layout, epi, K);
    GemmBatch b = b_in;
    b.split_ways = 0;
    int per_xcd = 0;
    if (b.band) {
        const int tiles_m = (b.M[0] + BM - 1) / BM, tiles_n = (b.N[0] + tn_w - 1) / tn_w;
        per_xcd = ((tiles_m / 8 + GROUP_M - 1) / GROUP_M) * GROUP_M * tiles_n * b.count;
    } else {
        for (int g = 0; g < b.count; ++g)
            per_xcd += (((b.M[g] + BM - 1) / BM) * ((b.N[g] + tn_w - 1) / tn_w) + 7) / 8;
    }
    if (per_xcd == 0) return hipSuccess;
    int64_t workgroups = 8 * (int64_t)per_xcd;
    const int ways = split_ways(b, tn_w, workgroups, epi, K, out_bf16);
    if (ways > 1) {
        b.split_tail = (int)(workgroups % cu_count());
        b.split_from = (int)(workgroups - b.split_tail);
        b.split_ways = ways;
        workgroups = b.split_from + (int64_t)ways * b.split_tail;
    }
    if (hipError_t e = launch_tiles(b, tn_w, dim3((unsigned)workgroups), layout, epi, ldaux, K,
                                    out_bf16, stream))
        return e;
    if (ways < 2) return hipSuccess;
    hipLaunchKernelGGL(split_fixup_kernel, dim3(4 * b.split_tail), dim3(256), 0, stream, b, tn_w);
    return hipGetLastError();
}
}  // namespace

hipError_t gemm_bf16_grouped(const GemmBatch& batch, int layout, int epi, int64_t ldaux,
                             int64_t K, bool out_bf16, hipStream_t stream)
{
    if (batch.count > kMaxBatch || K <= 0) return hipErrorInvalidValue;
    if (batch.count <= 0) return hipSuccess;
    GemmBatch b = batch;
    b.band = 0;
    return launch(b, layout, epi, ldaux, K, out_bf16, stream);
}

hipError_t gemm_bf16_batched(const GemmBatch& batch, int layout, int epi, int64_t lda,
                             int64_t ldb, int64_t ldc, int64_t ldaux, int64_t M, int64_t N,
                             int64_t K, bool out_bf16, hipStream_t stream)
{
    if (batch.count > kMaxBatch || K <= 0) return hipErrorInvalidValue;
    if (M <= 0 || N <= 0 || batch.count <= 0) return hipSuccess;
    GemmBatch b = batch;
    for (int g = 0; g < b.count; ++g) {
        b.M[g] = (int)M;
        b.N[g] = (int)N;
        b.lda[g] = lda;
        b.ldb[g] = ldb;
        b.ldc[g] = ldc;
    }
    const int tiles_m = (int)((M + BM - 1) / BM);
    bool shared_a = b.count > 1;
    for (int i = 1; i < b.count; ++i) shared_a = shared_a && b.A[i] == b.A[0];
    b.band = (shared_a && tiles_m % 8 == 0) ? 1 : 0;
    return launch(b, layout, epi, ldaux, K, out_bf16, stream);
}

hipError_t gemm_bf16_batched(const GemmBatch& batch, int64_t lda, int64_t ldb, int64_t ldc,
                             int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                             hipStream_t stream)
{
    return gemm_bf16_batched(batch, GEMM_NN, gelu ? EPI_GELU : EPI_NONE, lda, ldb, ldc, 0, M, N,
                             K, out_bf16, stream);
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

