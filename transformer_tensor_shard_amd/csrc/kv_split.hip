// Attention with Q, K and V split along the feature dimension over P ranks
// ("strategy B", K/V splitting, of the ops-transformer article
// (intelliparadigm.com/article/weixin_42537919/2252113) §3.1): rank r holds
// the features F_r = [r·d/P, (r+1)·d/P) of every head's Q, K and V, computes
// the partial scores S_r = Q_r·K_r^T, the partial scores are summed over the
// ranks (the softmax is not linear, so the sum comes first), and rank r forms
// its feature slice of the output, O[:, F_r] = softmax(S/sqrt(d) + mask)·V_r.
// On one GPU, per (sequence, head) pair:
//  * the P partial-score products are NT GEMMs with K = d/P (f32 out, one
//    [s, s] matrix per rank), in grouped launches; under the causal mask the
//    256x256 tiles that lie wholly past the diagonal are skipped (no query
//    reads them);
//  * kv_softmax_kernel sums a query row's P partial rows in rank order,
//    scales, masks, and writes the unnormalised weights e = 2^(x - max) in
//    bf16 (the largest is exactly 1) and the sum of those same rounded
//    weights (HBM bound: P·s f32 read and s bf16 written per row);
//  * O = e·V is one NN GEMM per pair with N = d (f32 out): its column block
//    F_r is exactly rank r's product with V_r (each output column depends
//    only on its own column of V), so the ranks' slices are formed side by
//    side; kv_normalize_kernel divides each row by its sum and rounds to
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

// One workgroup per query row t of chunk pair p: parts [n][P][s][s] f32,
// weights [n][s][s] bf16, rowsum [n][s] f32.  Keys past the diagonal
// (causal) are neither read nor given weight.
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
    const int64_t ss = (int64_t)s * s;
    const float* base = parts + p * P * ss + (int64_t)t * s;
    f32x4 acc[KV_MAXV];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KV_MAXV; ++i) {
        const int c = threadIdx.x + 256 * i;
        acc[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (c >= nv || (causal && 4 * c > t)) continue;
        f32x4 v = __builtin_nontemporal_load((const f32x4*)base + c);
        for (int r = 1; r < P; ++r) v += __builtin_nontemporal_load((const f32x4*)(base + r * ss) + c);
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
    return n * s * s * (4 * (int64_t)P + 2) + n * s * (4 * d + 4);
}

hipError_t kv_split_attention(const __bf16* qkv, int64_t ld, __bf16* O, int64_t ldo, int b, int s,
                              int H, int d, int P, bool causal, void* ws, hipStream_t stream)
{
    const int pairs = b * H, w = d / P;
    const int64_t ss = (int64_t)s * s;
    const int64_t HD = (int64_t)H * d;
    // workspace: partial scores [n][P][s][s] f32, then e·V [n][s][d] f32 and
    // the row sums [n][s] f32, then the weights [n][s][s] bf16
    float* parts = (float*)ws;
    const int64_t n_max = pairs < kKvChunk ? pairs : kKvChunk;
    float* accv = parts + n_max * P * ss;
    float* rowsum = accv + n_max * s * d;
    __bf16* probs = (__bf16*)(rowsum + n_max * s);
    const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    for (int p0 = 0; p0 < pairs; p0 += kKvChunk) {
        const int n = pairs - p0 < kKvChunk ? pairs - p0 : kKvChunk;
        // the partial scores of every rank of the chunk's pairs
        GemmBatch gb = {};
        gb.skip_upper = causal ? 1 : 0;
        for (int k = 0; k < n * P; ++k) {
            const int i = k / P, r = k % P, pair = p0 + i;
            const int64_t seq = (int64_t)(pair / H) * s * ld, head = (int64_t)(pair % H) * d;
            const int g = gb.count++;
            gb.A[g] = qkv + seq + head + r * w;
            gb.B[g] = qkv + seq + HD + head + r * w;
            gb.C[g] = parts + (int64_t)k * ss;
            gb.M[g] = s;
            gb.N[g] = s;
            gb.lda[g] = ld;
            gb.ldb[g] = ld;
            gb.ldc[g] = s;
            if (gb.count == kMaxBatch || k + 1 == n * P) {
                if (hipError_t e = gemm_bf16_grouped(gb, GEMM_NT, EPI_NONE, 0, w, false, stream))
                    return e;
                gb = GemmBatch{};
                gb.skip_upper = causal ? 1 : 0;
            }
        }
        hipLaunchKernelGGL(kv_softmax_kernel, dim3((unsigned)(n * (int64_t)s)), dim3(256), 0,
                           stream, (const float*)parts, P, s, causal ? 1 : 0, scale_log2, probs,
                           rowsum);
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
