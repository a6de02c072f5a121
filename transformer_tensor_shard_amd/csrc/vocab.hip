// The two vocabulary ends of the model, vocab-parallel ("图解Transformer并行计算"
// §4.1, §4.2):
//  * input embedding: rank r holds rows [vstart, vstart + V_r) of the table
//    E [V, h]; a token in that range gets its row, any other token a zero
//    row, and the sum over ranks (the all-reduce) is the full lookup.  One
//    256-thread workgroup per token row, 16-byte loads and stores;
//  * cross-entropy: the logits H·E_r^T come from the MFMA GEMM with the
//    CE-statistics epilogue (gemm_bf16.hip), which leaves per row and
//    128-column piece t the maximum m_t and sum_j exp(l_j - m_t), and the
//    target's logit.  Here, in the stable form: the rank's row statistics
//        m_r = max_t m_t,   s_r = sum_t s_t·exp(m_t - m_r)   (pieces in order);
//    the cross-rank combine (the all-reduces of the max, the exp-sum and the
//    target logit) and the loss
//        m = max_r m_r,  s = sum_r s_r·exp(m_r - m),  t = sum_r t_r,
//        loss = log(s) + m - t   (= -log softmax(target));
//    and the mean over tokens by one workgroup in a fixed order.  Every sum is
//    taken in an order fixed by the shape, so results are reproducible.
#include "tp_kernels.h"

#include <math.h>

namespace tpk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void embed_shard_kernel(const int* __restrict__ tokens,
                                                          const __bf16* __restrict__ E,
                                                          int64_t V_r, int64_t h, int64_t vstart,
                                                          void* __restrict__ out, int out_bf16)
{
    const int64_t row = blockIdx.x;
    const int64_t local = (int64_t)tokens[row] - vstart;
    const bool mine = local >= 0 && local < V_r;
    const __bf16* src = E + (mine ? local : 0) * h;
    for (int64_t u = threadIdx.x; u < h / 8; u += 256) {
        bf16x8 v = {};
        if (mine) v = *(const bf16x8*)(src + u * 8);
        if (out_bf16) {
            *(bf16x8*)((__bf16*)out + row * h + u * 8) = v;
        } else {
            float* o = (float*)out + row * h + u * 8;
            *(f32x4*)o = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
            *(f32x4*)(o + 4) = f32x4{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// piece statistics [M][ntn][2] -> the rank's m_r, s_r (stats[0..M), stats[M..2M))
__global__ __launch_bounds__(256) void ce_rank_reduce_kernel(const float* __restrict__ tiles,
                                                             int ntn, int64_t M,
                                                             float* __restrict__ stats)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= M) return;
    const float* t = tiles + row * ntn * 2;
    float m = -INFINITY;
    for (int j = 0; j < ntn; ++j) m = fmaxf(m, t[2 * j]);
    float s = 0.0f;
    for (int j = 0; j < ntn; ++j) s += t[2 * j + 1] * expf(t[2 * j] - m);
    stats[row] = m;
    stats[M + row] = s;
}

// ranks' [3][M] statistics (m_r, s_r, t_r), rank r at stats + r·3M -> loss [M]
__global__ __launch_bounds__(256) void ce_combine_kernel(const float* __restrict__ stats, int P,
                                                         int64_t M, float* __restrict__ loss)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= M) return;
    float m = -INFINITY;
    for (int r = 0; r < P; ++r) m = fmaxf(m, stats[r * 3 * M + row]);
    float s = 0.0f, t = 0.0f;
    for (int r = 0; r < P; ++r) {
        const float* st = stats + r * 3 * M;
        s += st[M + row] * expf(st[row] - m);
        t += st[2 * M + row];
    }
    loss[row] = logf(s) + m - t;
}

// mean of x[0..n) by one workgroup: thread i sums x[i], x[i+256], ... in
// order, then a fixed tree over the 256 partial sums
__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int64_t n,
                                                   float* __restrict__ out)
{
    __shared__ float part[256];
    float acc = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += 256) acc += x[i];
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = part[0] / (float)n;
}

inline unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t embed_shard(const int* tokens, int64_t M, const void* E_r, int64_t V_r, int64_t h,
                       int64_t vstart, void* out, bool out_bf16, hipStream_t stream)
{
    hipLaunchKernelGGL(embed_shard_kernel, dim3((unsigned)M), dim3(256), 0, stream, tokens,
                       (const __bf16*)E_r, V_r, h, vstart, out, out_bf16 ? 1 : 0);
    return hipGetLastError();
}

hipError_t fill_zero(float* p, int64_t n, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks(n)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t ce_rank_reduce(const float* tiles, int ntn, int64_t M, float* stats, hipStream_t stream)
{
    hipLaunchKernelGGL(ce_rank_reduce_kernel, dim3(blocks(M)), dim3(256), 0, stream, tiles, ntn,
                       M, stats);
    return hipGetLastError();
}

hipError_t ce_combine(const float* stats, int P, int64_t M, float* loss, float* loss_mean,
                      hipStream_t stream)
{
    hipLaunchKernelGGL(ce_combine_kernel, dim3(blocks(M)), dim3(256), 0, stream, stats, P, M,
                       loss);
    if (loss_mean)
        hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, stream, (const float*)loss, M,
                           loss_mean);
    return hipGetLastError();
}

}  // namespace tpk
