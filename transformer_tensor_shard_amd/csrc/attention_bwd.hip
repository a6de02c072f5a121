// Backward of the head-sharded attention core for gfx950, d = 128
// ("图解Transformer并行计算" §3.2, backward: each rank computes the gradients
// of its own heads from the same upstream gradient).  Per (sequence, head),
// with S = Q·K^T/sqrt(d) (causal keys masked), P = softmax(S) recomputed from
// the forward's log2 normaliser L (P = 2^(S·log2(e) - L)) and dO the upstream
// gradient:
//     D_q = sum_d dO·O  (= sum_k P·dP per query),   dP = dO·V^T,
//     dS = P ⊙ (dP - D),   dQ = dS·K/sqrt(d),   dK = dS^T·Q/sqrt(d),   dV = P^T·dO.
//
// Two kernels, no atomics, so the result is bitwise reproducible:
//  * query-stationary (dQ): one workgroup of 4 waves = 128 queries of one
//    (sequence, head); each wave holds Q and dO of its 32 queries in
//    registers as MFMA B operands.  64-key K/V tiles stream through LDS.  Per
//    32-key half of a tile a wave computes S^T = K·Q^T and dP^T = V·dO^T
//    (MFMA 32x32x16, A = K/V rows read from LDS), so every lane holds one
//    query's column and P, dS are lane-local; then dQ^T += K^T·dS^T with K^T
//    from the LDS transpose read.  It also forms D_q from dO and O and
//    stores it for the second kernel;
//  * key-stationary (dK, dV): one workgroup = 128 keys, each wave holding K
//    and V of its 32 keys in registers; 64-query tiles of Q and dO (plus the
//    tile's L and D) stream through LDS.  Per 32-query half a wave computes
//    S = Q·K^T and dP = dO·V^T (each lane one key's column), P and dS
//    element-wise, then dV^T += dO^T·P and dK^T += Q^T·dS with dO^T and Q^T
//    from transpose reads.
// Tiles reach LDS by the gfx950 direct-to-LDS buffer loads (no staging
// registers); a buffer range that ends at the sequence's last row zero-fills
// rows past it.  Two LDS stages, each its own array: loads of the next tile
// overlap this tile's MFMAs and every LDS address is static.  The causal mask
// (and the sequence end) is applied only on tiles that reach them, by setting
// the masked scores to -inf before the exponential.
// When an accumulator feeds the next MFMA as its B operand, the lane's eight
// k values are rows {4h..4h+3, 8+4h..8+4h+3} of a 16-row step (h = lane/32),
// and the A operand's transpose reads take the same rows, so nothing is
// shuffled between lanes.
#include "tp_kernels.h"

#include <math.h>

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int D = 128, NW = 4, NT = 64 * NW;
constexpr int BQ = 32 * NW;          // queries per dQ workgroup
constexpr int BK = 32 * NW;          // keys per dK/dV workgroup
constexpr int T64 = 64;              // rows per streamed tile
constexpr int TILE = T64 * D * 2;    // 16 KiB: 64 rows x 256 B
constexpr unsigned OOB = 0x80000000u;
constexpr int VMCNT0 = 0x0F70;       // s_waitcnt vmcnt(0)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                             0x00020000);
}

// Tile swizzle: logical 16-byte unit u of row r sits at physical unit
// u ^ swz(r).  Over 16 consecutive rows swz takes 16 distinct values (the
// 16-byte row reads of one unit by 16 lanes hit distinct banks), and rows
// 4j..4j+3 differ in bits 2-3 (the four rows a transpose read of 32 columns
// touches land in four distinct 64-byte windows).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// byte offset of element (row, col) in a [rows][128] bf16 tile
__device__ __forceinline__ unsigned tile_off(int row, int col) {
    return row * 256 + (((col >> 3) ^ swz(row)) << 4) + (col & 7) * 2;
}

// Direct-to-LDS copy of a 64 x 128 bf16 tile: wave w fills the 1 KiB chunks
// 4w..4w+3 (rows 4c..4c+3 of chunk c); lane l fetches row 4c + l/16, logical
// unit (l % 16) ^ swz(row), so the tile lands swizzled.  `voff[j]` is the
// lane's loop-invariant byte offset for chunk 4w + j relative to the tile's
// first row and column; the resource's range ends at the sequence's end.
__device__ __forceinline__ unsigned dma_voff(int w, int j, int lane, int64_t ld) {
    const int c = 4 * w + j;
    const int r = 4 * c + (lane >> 4);
    const int lu = (lane & 15) ^ swz(r);
    return (unsigned)((int64_t)r * ld + lu * 8) * 2u;
}
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, char* tile, const unsigned (&voff)[4],
                                         int w) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, tile + (4 * w + j) * 1024), 16,
                                                 voff[j], 0, 0, 0);
}
// resource for rows row0.. of a [s, ld] bf16 sequence, starting at column col
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const __bf16* seq, int64_t ld, int row0,
                                                            int col, int s) {
    const int64_t bytes = (int64_t)(s - row0) * ld * 2;
    return make_rsrc(seq + (int64_t)row0 * ld + col,
                     __builtin_amdgcn_readfirstlane(bytes <= 0 ? 0 : (int)(bytes < 0x7ffffff0 ? bytes : 0x7ffffff0)));
}

// MFMA A operand "rows of the tile transposed": lane (h = lane/32, column
// lane & 31 of a 32-wide block) receives the 8 values of rows
// {4h..4h+3, 8+4h..8+4h+3} -- the k order of a B operand taken from an
// accumulator.  lo/hi are the lane's addresses of the two 4-row reads.
__device__ __forceinline__ bf16x8 tr_read(const char* base, unsigned lo, unsigned hi) {
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base + lo));
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, base + hi));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// stage a wave's [128 dims x 32 rows] f32 accumulator (acc[dt][r] holds dim
// 32dt + 8(r>>2) + 4h + (r&3) of row lane&31) as bf16 rows of 256 B, times
// `mul`; 32 rows x 256 B at `stage` (16-byte units XOR-ed by row & 15)
__device__ __forceinline__ void stage_rows(char* stage, const f32x16 (&acc)[4], float mul,
                                           int l32, int h) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[dt][4 * rq + e] * mul);
            const int d0 = 32 * dt + 8 * rq + 4 * h;
            *(bf16x4*)(stage + l32 * 256 + (((d0 >> 3) ^ (l32 & 15)) << 4) + (d0 & 7) * 2) = v;
        }
}

// write 32 staged rows to dst rows row0.., columns col..col+127 (ld elements)
__device__ __forceinline__ void store_rows(const char* stage, __bf16* dst, int64_t ld, int row0,
                                           int nrows_valid, int col, int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = i * 64 + lane;
        const int row = idx >> 4, unit = idx & 15;
        const u32x4 v = *(const u32x4*)(stage + row * 256 + ((unit ^ (row & 15)) << 4));
        if (row < nrows_valid) *(u32x4*)(dst + (int64_t)(row0 + row) * ld + col + unit * 8) = v;
    }
}

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.0f;
}

// --------------------------------------------------------------------- dQ
__global__ __launch_bounds__(NT, 1) void attn_bwd_dq_kernel(
    const __bf16* __restrict__ qkv, int64_t ld, const __bf16* __restrict__ O,
    const __bf16* __restrict__ dO, int64_t ldo, const float* __restrict__ lse,
    float* __restrict__ Dvec, __bf16* __restrict__ dqkv, int64_t ldd, int s, int Hl, int nqb,
    int n_bh, int causal, float scale_log2, float scale)
{
    // one stage = K tile then V tile
    __shared__ __attribute__((aligned(1024))) char lds0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) char lds1[2 * TILE];

    // all query blocks of a (sequence, head) on one XCD, heaviest first
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int bh = (local / nqb) * 8 + xcd;
    if (bh >= n_bh) return;
    const int qb = nqb - 1 - local % nqb;
    const int beta = bh / Hl, head = bh % Hl;
    const int q0 = qb * BQ;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    const __bf16* seq = qkv + (int64_t)beta * s * ld;
    const int qcol = head * D, kcol = Hl * D + head * D, vcol = 2 * Hl * D + head * D;
    const int64_t stat = ((int64_t)beta * Hl + head) * s;

    // Q and dO of the lane's query as B operands (dims 16kk + 8h .. +7), and
    // D_q = sum over the head's dims of dO·O
    const int my_q = q0 + 32 * w + l32;
    const bool qok = my_q < s;
    bf16x8 qf[8], dof[8];
    float dsum = 0.0f;
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(seq, 0x7ffffff0);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + (int64_t)beta * s * ldo, 0x7ffffff0);
        const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + (int64_t)beta * s * ldo, 0x7ffffff0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const unsigned qoff = qok ? (unsigned)((int64_t)my_q * ld + qcol + kk * 16 + 8 * h) * 2u : OOB;
            const unsigned ooff = qok ? (unsigned)((int64_t)my_q * ldo + head * D + kk * 16 + 8 * h) * 2u : OOB;
            qf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, 0, 0));
            dof[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, ooff, 0, 0));
            const bf16x8 of = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, ooff, 0, 0));
#pragma unroll
            for (int e = 0; e < 8; ++e) dsum = fmaf((float)dof[kk][e], (float)of[e], dsum);
        }
    }
    const float Dq = dsum + __shfl_xor(dsum, 32);
    if (qok && h == 0) Dvec[stat + my_q] = Dq;
    const float L2 = qok ? lse[stat + my_q] : 0.0f;

    unsigned voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) voff[j] = dma_voff(w, j, lane, ld);
    auto dma_kv = [&](char* stage, int kv0) {
        dma_tile(rows_rsrc(seq, ld, kv0, kcol, s), stage, voff, w);
        dma_tile(rows_rsrc(seq, ld, kv0, vcol, s), stage + TILE, voff, w);
    };
    // row reads (A = K or V rows 32t + l32, dims 16kk + 8h..)
    unsigned rd[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) rd[kk] = tile_off(l32, 16 * kk + 8 * h);
    // transpose reads of K (A = K^T: dims 32dt + (lane & 31), keys in B order)
    const int G = lane >> 4, gi = lane & 15;
    unsigned tlo[4], thi[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const int col = 32 * dt + 16 * (G & 1) + 4 * (gi & 3);
        tlo[dt] = tile_off(4 * h + (gi >> 2), col);
        thi[dt] = tile_off(8 + 4 * h + (gi >> 2), col);
    }

    f32x16 dq[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) zero(dq[dt]);

    const int kv_end = causal ? min(s, q0 + BQ) : s;
    const int n_kv = (kv_end + T64 - 1) / T64;
    const int qw_lo = q0 + 32 * w, qw_hi = qw_lo + 31;
    const int lim = causal ? min(my_q, s - 1) : s - 1;

    auto compute = [&](const char* base, int kv0) {
        if (causal && kv0 > qw_hi) return;          // every key after the wave's queries
        const bool edge = (causal && kv0 + T64 - 1 > qw_lo) || kv0 + T64 > s;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x16 sacc, pacc;
            zero(sacc);
            zero(pacc);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const bf16x8 kf = *(const bf16x8*)(base + rd[kk] + t * 32 * 256);
                const bf16x8 vf = *(const bf16x8*)(base + TILE + rd[kk] + t * 32 * 256);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc, 0, 0, 0);
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[kk], pacc, 0, 0, 0);
            }
            if (edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                    sacc[r] = key > lim ? -INFINITY : sacc[r];
                }
            }
            bf16x8 dsk[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -L2));
                dsk[r >> 3][r & 7] = (__bf16)(p * (pacc[r] - Dq));
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const char* kb_base = base + (32 * t + 16 * half) * 256;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        tr_read(kb_base, tlo[dt], thi[dt]), dsk[half], dq[dt], 0, 0, 0);
            }
        }
    };
    // tile i in stage (i & 1); the barrier after a tile publishes the next
    // tile's LDS and frees the one just read
    auto step = [&](char* cur, char* nxt, int i) {
        if (i + 1 < n_kv) dma_kv(nxt, (i + 1) * T64);
        compute(cur, i * T64);
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        __syncthreads();
    };
    dma_kv(lds0, 0);
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    __syncthreads();
    for (int i = 0; i < n_kv; i += 2) {
        step(lds0, lds1, i);
        if (i + 1 < n_kv) step(lds1, lds0, i + 1);
    }

    char* stage = lds0 + w * (32 * 256);
    stage_rows(stage, dq, scale, l32, h);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    store_rows(stage, dqkv + (int64_t)beta * s * ldd, ldd, qw_lo, s - qw_lo, qcol, lane);
}

// ------------------------------------------------------------------ dK, dV
constexpr int STAGE_KV = 2 * TILE + 512;     // Q tile, dO tile, L[64], D[64]

__global__ __launch_bounds__(NT, 2) void attn_bwd_dkv_kernel(
    const __bf16* __restrict__ qkv, int64_t ld, const __bf16* __restrict__ dO, int64_t ldo,
    const float* __restrict__ lse, const float* __restrict__ Dvec, __bf16* __restrict__ dqkv,
    int64_t ldd, int s, int Hl, int nkb, int n_bh, int causal, float scale_log2, float scale)
{
    __shared__ __attribute__((aligned(1024))) char lds0[STAGE_KV];
    __shared__ __attribute__((aligned(1024))) char lds1[STAGE_KV];

    // all key blocks of a (sequence, head) on one XCD; key block 0 (under a
    // causal mask the one with the most query tiles) first
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int bh = (local / nkb) * 8 + xcd;
    if (bh >= n_bh) return;
    const int kb = local % nkb;
    const int beta = bh / Hl, head = bh % Hl;
    const int k0 = kb * BK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    const __bf16* seq = qkv + (int64_t)beta * s * ld;
    const __bf16* dseq = dO + (int64_t)beta * s * ldo;
    const int qcol = head * D, kcol = Hl * D + head * D, vcol = 2 * Hl * D + head * D;
    const int64_t stat = ((int64_t)beta * Hl + head) * s;

    // K and V of the lane's key as B operands
    const int kw0 = k0 + 32 * w;
    const int my_k = kw0 + l32;
    bf16x8 kf[8], vf[8];
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(seq, 0x7ffffff0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const unsigned off = (unsigned)((int64_t)my_k * ld + kk * 16 + 8 * h) * 2u;
            kf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs, my_k < s ? off + kcol * 2u : OOB, 0, 0));
            vf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs, my_k < s ? off + vcol * 2u : OOB, 0, 0));
        }
    }

    // the tile's Q, dO, and (wave 0) its 64 L and 64 D values as f32; the
    // lane offsets are recomputed per tile (a few integer operations) rather
    // than held in registers across the loop
    auto dma_q = [&](char* stage, int q0) {
        // the empty asm makes the lane index opaque here, so the compiler
        // cannot hoist these offsets out of the tile loop (where it spilled
        // them to scratch and reloaded them every tile)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        unsigned voff_q[4], voff_o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            voff_q[j] = dma_voff(w, j, ln, ld);
            voff_o[j] = dma_voff(w, j, ln, ldo);
        }
        dma_tile(rows_rsrc(seq, ld, q0, qcol, s), stage, voff_q, w);
        dma_tile(rows_rsrc(dseq, ldo, q0, head * D, s), stage + TILE, voff_o, w);
        if (w == 0) {
            const int bytes = __builtin_amdgcn_readfirstlane(4 * (s - q0));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(lse + stat + q0, bytes),
                                                     LDS_PTR(void, stage + 2 * TILE), 4,
                                                     4u * lane, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(Dvec + stat + q0, bytes),
                                                     LDS_PTR(void, stage + 2 * TILE + 256), 4,
                                                     4u * lane, 0, 0, 0);
        }
    };

    f32x16 dk[4], dv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        zero(dk[dt]);
        zero(dv[dt]);
    }

    auto compute = [&](const char* base, int q0) {
        if (causal && q0 + T64 - 1 < kw0) return;   // every query before the wave's keys
        // LDS read addresses, derived per tile from an opaque lane index: held
        // across the loop they pushed two K/V fragments out to scratch.
        // Row reads: dims 16kk + 8h of row 32t + l32 sit at rd0 ^ (kk << 5)
        // (the unit index 2kk + h XOR-ed by swz(l32); kk moves only unit bits
        // 1-3); transpose reads of 4 key rows x 16 dims per 16-lane group.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const unsigned rd0 = tile_off(ln & 31, 8 * (ln >> 5));
        const int G = ln >> 4, gi = ln & 15, hh = ln >> 5;
        unsigned tlo[4], thi[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int col = 32 * dt + 16 * (G & 1) + 4 * (gi & 3);
            tlo[dt] = tile_off(4 * hh + (gi >> 2), col);
            thi[dt] = tile_off(8 + 4 * hh + (gi >> 2), col);
        }
        const float* Ls = (const float*)(base + 2 * TILE);
        const float* Ds = Ls + T64;
        const bool edge = (causal && q0 < kw0 + 31) || q0 + T64 > s;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x16 sacc, pacc;
            zero(sacc);
            zero(pacc);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const unsigned rd = rd0 ^ (kk << 5);
                const bf16x8 qa = *(const bf16x8*)(base + rd + t * 32 * 256);
                const bf16x8 da = *(const bf16x8*)(base + TILE + rd + t * 32 * 256);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], sacc, 0, 0, 0);
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kk], pacc, 0, 0, 0);
            }
            if (edge) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = q0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                    sacc[r] = (q >= s || (causal && q < my_k)) ? -INFINITY : sacc[r];
                }
            }
            // P and dS of both 16-query steps (accumulator elements 8·half ..
            // +7) first, so that the f32 scores are dead before the dV and dK
            // MFMAs (keeping them live across those spilled a K/V fragment)
            bf16x8 pk[2], dsk[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int rq2 = 0; rq2 < 2; ++rq2) {
                    const int rq4 = 2 * half + rq2;
                    const int qi = 32 * t + 8 * rq4 + 4 * h;   // tile query of element e = 0
                    const f32x4 Lv = *(const f32x4*)(Ls + qi);
                    const f32x4 Dv = *(const f32x4*)(Ds + qi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * rq4 + e;
                        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -Lv[e]));
                        pk[half][r & 7] = (__bf16)p;
                        dsk[half][r & 7] = (__bf16)(p * (pacc[r] - Dv[e]));
                    }
                }
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const char* qb_base = base + (32 * t + 16 * half) * 256;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        tr_read(qb_base + TILE, tlo[dt], thi[dt]), pk[half], dv[dt], 0, 0, 0);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        tr_read(qb_base, tlo[dt], thi[dt]), dsk[half], dk[dt], 0, 0, 0);
                }
            }
        }
    };
    const int qt0 = causal ? k0 / T64 : 0;
    const int nqt = (s + T64 - 1) / T64;
    auto step = [&](char* cur, char* nxt, int qt) {
        if (qt + 1 < nqt) dma_q(nxt, (qt + 1) * T64);
        compute(cur, qt * T64);
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        __syncthreads();
    };
    dma_q(lds0, qt0 * T64);
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    __syncthreads();
    for (int qt = qt0; qt < nqt; qt += 2) {
        step(lds0, lds1, qt);
        if (qt + 1 < nqt) step(lds1, lds0, qt + 1);
    }

    // dK and dV staged in the two (idle) stages, 8 KiB per wave each
    char* stage_k = lds0 + w * (32 * 256);
    char* stage_v = lds1 + w * (32 * 256);
    stage_rows(stage_k, dk, scale, l32, h);
    stage_rows(stage_v, dv, 1.0f, l32, h);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    __bf16* rows = dqkv + (int64_t)beta * s * ldd;
    store_rows(stage_k, rows, ldd, kw0, s - kw0, kcol, lane);
    store_rows(stage_v, rows, ldd, kw0, s - kw0, vcol, lane);
}

}  // namespace

hipError_t attention_bwd(const void* qkv, int64_t ld_qkv, const void* O, const void* dO,
                         const float* lse, float* Dvec, void* dqkv, int64_t b, int64_t s,
                         int64_t H_l, bool causal, hipStream_t stream)
{
    const int n_bh = (int)(b * H_l);
    const int groups_per_xcd = (n_bh + 7) / 8;
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const float scale = (float)(1.0 / sqrt((double)D));
    const int nqb = (int)((s + BQ - 1) / BQ), nkb = (int)((s + BK - 1) / BK);
    const int64_t ldo = H_l * D, ldd = 3 * H_l * D;
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3(8 * groups_per_xcd * nqb), dim3(NT), 0, stream,
                       (const __bf16*)qkv, ld_qkv, (const __bf16*)O, (const __bf16*)dO, ldo, lse,
                       Dvec, (__bf16*)dqkv, ldd, (int)s, (int)H_l, nqb, n_bh, causal ? 1 : 0,
                       scale_log2, scale);
    hipLaunchKernelGGL(attn_bwd_dkv_kernel, dim3(8 * groups_per_xcd * nkb), dim3(NT), 0, stream,
                       (const __bf16*)qkv, ld_qkv, (const __bf16*)dO, ldo, lse,
                       (const float*)Dvec, (__bf16*)dqkv, ldd, (int)s, (int)H_l, nkb, n_bh,
                       causal ? 1 : 0, scale_log2, scale);
    return hipGetLastError();
}

}  // namespace tpk
