// Attention with Q, K and V split along the feature dimension over P ranks
// ("strategy B", K/V splitting, of the ops-transformer article
// (intelliparadigm.com/article/weixin_42537919/2252113) §3.1): rank r holds
// the features F_r = [r·d/P, (r+1)·d/P) of every head's Q, K and V, computes
// the partial scores S_r = Q_r·K_r^T, the partial scores are summed over the
// ranks (the softmax is not linear, so the sum comes first), and rank r forms
// its feature slice of the output, O[:, F_r] = softmax(S/sqrt(d) + mask)·V_r.
// On one GPU, per (sequence, head) pair:
//  * kv_scores_kernel forms the P partial-score products, K = d/P (f32 out,
//    one [s, s] matrix per rank, stored as 128x128 tiles), operands loaded
//    straight into registers;
//    under the causal mask the 128x128 tiles that lie wholly past the
//    diagonal are skipped (no query reads them);
//  * kv_softmax_kernel sums a query row's P partial rows in rank order,
//    scales, masks, and writes the unnormalised weights e = 2^(x - max) in
//    bf16 (the largest is exactly 1) and the sum of those same rounded
//    weights (HBM bound: P·s f32 read and s bf16 written per row);
//  * O = e·V is one NN GEMM per pair with N = d (f32 out): its column block
//    F_r is exactly rank r's product with V_r (each output column depends
//    only on its own column of V), so the ranks' slices are formed side by
//    side (under the causal mask a row tile's K loop stops at its last row:
//    the weights past the diagonal are zero); kv_normalize_kernel divides
//    each row by its sum and rounds to
//    bf16 once.  The weights applied to V thus sum to one exactly, as in the
//    head-sharded attention kernel.
// Pairs are processed in chunks of kKvChunk, the workspace holding one
// chunk's partial scores and probabilities.
#include "tp_kernels.h"

#include <math.h>

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int KV_MAXV = kKvMaxS / (256 * 4);     // float4 units per thread

__device__ __forceinline__ float wg_reduce(float v, float* red, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float u = __shfl_xor(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();                 // red[] may still be read by a previous call
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < 4; ++i) t = is_max ? fmaxf(t, red[i]) : t + red[i];
    return t;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr unsigned KV_OOB = 0x80000000u;     // buffer offset past any range: reads 0

// A partial-score matrix is stored tile by tile: 128x128 f32 tiles in
// row-major tile order, each tile row-major in 64 KiB of its own (a ragged
// last tile row or column padded), so that the workgroup forming a tile
// writes one contiguous block instead of 128 row pieces 4·s bytes apart.
__host__ __device__ inline int64_t kv_part_floats(int64_t s) {
    const int64_t nt = (s + 127) / 128;
    return nt * nt * 16384;
}
__device__ __forceinline__ int64_t kv_part_index(int s, int row, int key) {
    const int nt = (s + 127) / 128;
    return ((int64_t)(row >> 7) * nt + (key >> 7)) * 16384 + (row & 127) * 128 + (key & 127);
}

// Partial scores of a small feature slice: S_r = Q_r·K_r^T, [s, s] f32 per
// (chunk pair, rank) in 128x128 tiles, w = d/P <= 128 features.  One workgroup of 4 waves per
// 128x128 tile (wave: 64 query rows x 64 keys as 4x4 MFMA 16x16x32 blocks).
// With a K of one to four 32-wide steps there is nothing to stage: each lane
// loads its MFMA operand fragments (16 bytes of one row) straight from
// memory, features past w read as zeros, and each wave's f32 block is staged
// through 8 KiB of LDS (32 KiB per workgroup, so several workgroups share a
// CU and their stores overlap) and stored with the non-temporal hint in whole
// 256-byte row segments of the workgroup's 64 KiB tile.  Under the causal mask a tile wholly past the
// diagonal is not computed (no query reads it).
__global__ __launch_bounds__(256) void kv_scores_kernel(const __bf16* __restrict__ qkv, int64_t ld,
                                                        int s, int H, int d, int P, int pair0,
                                                        int causal, float* __restrict__ parts)
{
    const int ntiles = (s + 127) / 128;           // a ragged last tile is bounds-checked
    const int64_t id = blockIdx.x;
    const int tn = (int)(id % ntiles), tm = (int)((id / ntiles) % ntiles);
    const int64_t k = id / ((int64_t)ntiles * ntiles);      // chunk pair * P + rank
    if (causal && tn > tm) return;
    __shared__ __attribute__((aligned(16))) char stage[4][32 * 256];
    const int i = (int)(k / P), r = (int)(k % P), pair = pair0 + i;
    const int w = d / P;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int m0 = tm * 128 + (wv >> 1) * 64, n0 = tn * 128 + (wv & 1) * 64;
    const __bf16* base = qkv + (int64_t)(pair / H) * s * ld + (int64_t)(pair % H) * d + r * w;
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(base), (short)0, (int)((int64_t)s * ld * 2 < 0x7ffffff0 ? (int64_t)s * ld * 2 : 0x7ffffff0), 0x00020000);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(base + (int64_t)H * d), (short)0,
        (int)((int64_t)s * ld * 2 < 0x7ffffff0 ? (int64_t)s * ld * 2 : 0x7ffffff0), 0x00020000);
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    f32x4v acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    const int kq = 8 * (lane >> 4);                // this lane's 8 features of a 32-wide step
    for (int k0 = 0; k0 < w; k0 += 32) {
        const bool in_k = k0 + kq < w;
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int row = m0 + 16 * a + (lane & 15);
            const unsigned off = (in_k && row < s) ? (unsigned)(((int64_t)row * ld + k0 + kq) * 2) : KV_OOB;
            fa[a] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int key = n0 + 16 * b + (lane & 15);
            const unsigned off = (in_k && key < s) ? (unsigned)(((int64_t)key * ld + k0 + kq) * 2) : KV_OOB;
            fb[b] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    // Lane holds key (lane & 15) and query rows 4·(lane >> 4) + e of each
    // block.  The wave's 64x64 f32 block goes out through its own 8 KiB of
    // LDS in two passes of 32 rows, so that each store instruction writes four
    // whole 256-byte row segments (storing from the accumulators wrote 64-byte
    // segments, half of a 128-byte line each, at about half the write rate).
    // The 16-byte unit of a staged row is XOR-ed with bits 2-3 of the row:
    // the four row groups of one LDS write then hit distinct banks.  s % 8 == 0,
    // so a unit's four keys are all inside or all past the row's end.
    float* out = parts + k * kv_part_floats(s);
    char* const st = stage[wv];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = 16 * a2 + 4 * (lane >> 4) + e;      // row within the pass
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int unit = 4 * b + ((lane & 15) >> 2);
                    *(float*)(st + rl * 256 + ((unit ^ (((rl >> 2) & 3) << 2)) << 4) +
                              (lane & 3) * 4) = acc[2 * p + a2][b][e];
                }
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): the wave's writes are done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = i * 64 + lane, rl = idx >> 4, unit = idx & 15;
            const f32x4 v = *(const f32x4*)(st + rl * 256 + ((unit ^ (((rl >> 2) & 3) << 2)) << 4));
            const int row = m0 + 32 * p + rl, key = n0 + 4 * unit;
            if (row < s && key < s)
                __builtin_nontemporal_store(v, (f32x4*)(out + kv_part_index(s, row, key)));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);               // reads done before the next pass writes
        __builtin_amdgcn_wave_barrier();
    }
}

// One workgroup per query row t of chunk pair p: parts [n][P] tiled partial
// scores (kv_part_index), weights [n][s][s] bf16, rowsum [n][s] f32.  Keys past the diagonal
// (causal) are neither read nor given weight.
template <int PT>   // the rank count when known at compile time (loads all in flight), else 0
__global__ __launch_bounds__(256) void kv_softmax_kernel(const float* __restrict__ parts, int P,
                                                         int s, int causal, float scale_log2,
                                                         __bf16* __restrict__ probs,
                                                         float* __restrict__ rowsum)
{
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int64_t p = row / s;
    const int t = (int)(row % s);
    const int nv = s / 4;
    const int64_t ss = (int64_t)s * s, ps = kv_part_floats(s);
    const float* base = parts + p * P * ps;
    f32x4 acc[KV_MAXV];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KV_MAXV; ++i) {
        const int c = threadIdx.x + 256 * i;
        acc[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (c >= nv || (causal && 4 * c > t)) continue;
        const float* pc = base + kv_part_index(s, t, 4 * c);    // 4 keys of one tile row
        f32x4 v = __builtin_nontemporal_load((const f32x4*)pc);
        if constexpr (PT > 0) {
#pragma unroll
            for (int r = 1; r < PT; ++r)
                v += __builtin_nontemporal_load((const f32x4*)(pc + r * ps));
        } else {
            for (int r = 1; r < P; ++r)
                v += __builtin_nontemporal_load((const f32x4*)(pc + r * ps));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool keep = !causal || 4 * c + e <= t;
            acc[i][e] = keep ? v[e] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, acc[i][e]);
        }
    }
    mx = wg_reduce(mx, red, true);     // finite: key 0 is always visible
    float sum = 0.0f;
    bf16x4* out = (bf16x4*)(probs + p * ss + (int64_t)t * s);
#pragma unroll
    for (int i = 0; i < KV_MAXV; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= nv) continue;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] = (__bf16)exp2f(acc[i][e] - mx);      // exp2(-inf) = 0
            sum += (float)o[e];
        }
        out[c] = o;
    }
    sum = wg_reduce(sum, red, false);
    if (threadIdx.x == 0) rowsum[row] = sum;
}

// O[token, head cols] = bf16(acc[row] / rowsum[row]) for the chunk's rows;
// acc [n][s][d] f32.  One thread per 4 columns.
__global__ __launch_bounds__(256) void kv_normalize_kernel(const float* __restrict__ acc,
                                                           const float* __restrict__ rowsum,
                                                           int64_t rows, int d, int s, int H,
                                                           int pair0, __bf16* __restrict__ O,
                                                           int64_t ldo)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int units = d / 4;
    if (idx >= rows * units) return;
    const int64_t row = idx / units;
    const int c = (int)(idx % units) * 4;
    const int64_t i = row / s, t = row % s;
    const int pair = pair0 + (int)i;
    const float inv = 1.0f / rowsum[row];
    const f32x4 v = *(const f32x4*)(acc + row * d + c);
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)(v[e] * inv);
    *(bf16x4*)(O + ((int64_t)(pair / H) * s + t) * ldo + (int64_t)(pair % H) * d + c) = o;
}

}  // namespace

int64_t kv_split_workspace_bytes(int64_t pairs, int64_t s, int64_t d, int P) {
    const int64_t n = pairs < kKvChunk ? pairs : kKvChunk;
    return n * (4 * (int64_t)P * kv_part_floats(s) + 2 * s * s) + n * s * (4 * d + 4);
}

hipError_t kv_split_attention(const __bf16* qkv, int64_t ld, __bf16* O, int64_t ldo, int b, int s,
                              int H, int d, int P, bool causal, void* ws, hipStream_t stream)
{
    const int pairs = b * H, w = d / P;
    const int64_t ss = (int64_t)s * s;
    const int64_t HD = (int64_t)H * d;
    // workspace: partial scores [n][P] (tiled, kv_part_floats(s) each) f32, then e·V [n][s][d] f32 and
    // the row sums [n][s] f32, then the weights [n][s][s] bf16
    float* parts = (float*)ws;
    const int64_t n_max = pairs < kKvChunk ? pairs : kKvChunk;
    float* accv = parts + n_max * P * kv_part_floats(s);
    float* rowsum = accv + n_max * s * d;
    __bf16* probs = (__bf16*)(rowsum + n_max * s);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    for (int p0 = 0; p0 < pairs; p0 += kKvChunk) {
        const int n = pairs - p0 < kKvChunk ? pairs - p0 : kKvChunk;
        // the partial scores of every rank of the chunk's pairs
        const int64_t ntiles = (s + 127) / 128;
        hipLaunchKernelGGL(kv_scores_kernel, dim3((unsigned)(n * (int64_t)P * ntiles * ntiles)),
                           dim3(256), 0, stream, qkv, ld, s, H, d, P, p0, causal ? 1 : 0, parts);
        if (hipError_t e = hipGetLastError()) return e;
        const dim3 rows_grid((unsigned)(n * (int64_t)s));
#define TP_KVS(PT) hipLaunchKernelGGL(kv_softmax_kernel<PT>, rows_grid, dim3(256), 0, stream, \
                                      (const float*)parts, P, s, causal ? 1 : 0, scale_log2, \
                                      probs, rowsum)
        if (P == 1) TP_KVS(1);
        else if (P == 2) TP_KVS(2);
        else if (P == 4) TP_KVS(4);
        else if (P == 8) TP_KVS(8);
        else TP_KVS(0);
#undef TP_KVS
        if (hipError_t e = hipGetLastError()) return e;
        // e·V per pair, all ranks' feature slices side by side, then the
        // division by the row sums
        GemmBatch pv = {};
        for (int i = 0; i < n; ++i) {
            const int pair = p0 + i;
            const int64_t row0 = (int64_t)(pair / H) * s, head = (int64_t)(pair % H) * d;
            pv.A[i] = probs + i * ss;
            pv.B[i] = qkv + row0 * ld + 2 * HD + head;
            pv.C[i] = accv + (int64_t)i * s * d;
            pv.M[i] = s;
            pv.N[i] = d;
            pv.lda[i] = s;
            pv.ldb[i] = ld;
            pv.ldc[i] = d;
        }
        pv.count = n;
        pv.causal_k = causal ? 1 : 0;       // weights are zero past the diagonal
        if (hipError_t e = gemm_bf16_grouped(pv, GEMM_NN, EPI_NONE, 0, s, false, stream)) return e;
        const int64_t units = (int64_t)n * s * (d / 4);
        hipLaunchKernelGGL(kv_normalize_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                           stream, (const float*)accv, (const float*)rowsum, (int64_t)n * s, d, s,
                           H, p0, O, ldo);
        if (hipError_t e = hipGetLastError()) return e;
    }
    return hipSuccess;
}

}  // namespace tpk
