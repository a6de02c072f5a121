// HBM-bound steps of the path: LayerNorm and the partial sum.
//
// * LayerNorm (the pre-LN block's nn.LayerNorm(h), PyTorch tensor-parallel
//   tutorial section 3.3): rows up to 16384 wide run through the row-sum
//   kernel below (row in registers); wider rows use one 256-thread workgroup
//   per row; the row is read once from HBM with 16-byte loads into LDS as f32, the mean and the
//   population variance are two exact passes over LDS (no E[x^2]-E[x]^2
//   cancellation), and the bf16 result is written with 16-byte stores.
// * Partial sum (the all-reduce's arithmetic on one GPU, "图解Transformer并行计算"
//   §1.1 / §2.1: Z = Z1 + Z2 + ...): a grid-stride streaming kernel, 16-byte
//   loads of every rank's partial, f32 sum in ascending rank order, optional
//   bias and residual, one 16-byte (f32) or 8-byte (bf16) store per 4 outputs.
// * Row partial sum (the same sum, one 256-thread workgroup per row of length
//   h <= 16384, the row held in registers as 16-byte vectors, every rank's
//   row segment loaded before any add so each thread has a rank's loads in
//   flight at once), optionally followed by the next sub-layer's LayerNorm of
//   the summed row: x1 = residual + sum_r Z_r and LN(x1) in one pass over HBM,
//   the pre-LN block's "x + attention(norm1(x))" feeding "norm2".
#include "tp_kernels.h"

namespace tpk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();              // red[] may still be read by a previous call
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
    return t;
}

template <bool IN_BF16>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const void* __restrict__ x, __bf16* __restrict__ y, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, int h)
{
    extern __shared__ float row[];
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    float s = 0.0f;
    for (int c = threadIdx.x * 8; c < h; c += 256 * 8) {
        float v[8];
        if (IN_BF16) {
            const bf16x8 t = *(const bf16x8*)((const __bf16*)x + m * h + c);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
        } else {
            const f32x4 a = *(const f32x4*)((const float*)x + m * h + c);
            const f32x4 b = *(const f32x4*)((const float*)x + m * h + c + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) { row[c + e] = v[e]; s += v[e]; }
    }
    const float mean = block_sum(s, red) / (float)h;
    float q = 0.0f;
    for (int c = threadIdx.x * 8; c < h; c += 256 * 8)
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float d = row[c + e] - mean; q += d * d; }
    const float var = block_sum(q, red) / (float)h;
    const float inv = rsqrtf(var + eps);
    for (int c = threadIdx.x * 8; c < h; c += 256 * 8) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = (row[c + e] - mean) * inv;
            if (gamma) v *= gamma[c + e];
            if (beta) v += beta[c + e];
            o[e] = (__bf16)v;
        }
        *(bf16x8*)(y + m * h + c) = o;
    }
}

template <bool PART_BF16, bool RES_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void partial_sum_kernel(
    void* Z, const void* __restrict__ parts, int P, int64_t n4, int h,
    const float* __restrict__ bias, const void* res)
{
    // Z may alias res (both f32): each element is read before it is written,
    // by the same thread.
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int r = 0; r < P; ++r) {
            if (PART_BF16) {
                const bf16x4 t = ((const bf16x4*)parts)[r * n4 + i];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += (float)t[e];
            } else {
                const f32x4 t = __builtin_nontemporal_load(((const f32x4*)parts) + (r * n4 + i));
                acc += t;
            }
        }
        if (bias) {
            const int c = (int)((i * 4) % h);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += bias[c + e];
        }
        if (res) {
            if (RES_BF16) {
                const bf16x4 t = ((const bf16x4*)res)[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += (float)t[e];
            } else {
                acc += ((const f32x4*)res)[i];
            }
        }
        if (OUT_BF16) {
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[e];
            ((bf16x4*)Z)[i] = o;
        } else {
            ((f32x4*)Z)[i] = acc;
        }
    }
}

// RES: 0 none, 1 f32, 2 bf16.  The summation order is the one of
// partial_sum_kernel (ranks ascending, then bias, then residual), so both give
// bit-identical sums.  E is the number of consecutive elements a thread owns
// per unit: 4 with f32 partials (16-byte loads), 8 with bf16 partials or none
// (16-byte bf16 loads); h % E == 0.  Outputs are stored with the
// non-temporal hint (written once, read by a later launch): ~1.5% faster.
template <int E> struct vec_of;
template <> struct vec_of<4> {
    typedef float f __attribute__((ext_vector_type(4)));
    typedef __bf16 b __attribute__((ext_vector_type(4)));
};
template <> struct vec_of<8> {
    typedef float f __attribute__((ext_vector_type(8)));
    typedef __bf16 b __attribute__((ext_vector_type(8)));
};

template <bool PART_BF16, int RES, bool OUT_BF16, bool LN, int E>
__global__ __launch_bounds__(256) void row_sum_kernel(
    void* __restrict__ Z, const void* __restrict__ parts, int P, int64_t n_units, int h,
    const float* __restrict__ bias, const void* __restrict__ res,
    __bf16* __restrict__ y, const float* __restrict__ gamma, const float* __restrict__ beta,
    float eps)
{
    typedef typename vec_of<E>::f fv;
    typedef typename vec_of<E>::b bv;
    constexpr int MAXV = 16384 / (256 * E);       // units per thread: rows up to 16384 wide
    __shared__ float red[4];
    const int nv = h / E;
    const int64_t row0 = (int64_t)blockIdx.x * nv;  // first unit of the row
    fv acc[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[i][e] = 0.0f;
    for (int r = 0; r < P; ++r) {
        fv t[MAXV];
#pragma unroll
        for (int i = 0; i < MAXV; ++i) {
            const int c = threadIdx.x + 256 * i;
            if (c < nv) {
                const int64_t k = r * n_units + row0 + c;
                if constexpr (PART_BF16) {
                    const bv b = ((const bv*)parts)[k];
#pragma unroll
                    for (int e = 0; e < E; ++e) t[i][e] = (float)b[e];
                } else {
                    t[i] = __builtin_nontemporal_load((const fv*)parts + k);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < MAXV; ++i)
            if (threadIdx.x + 256 * i < nv) acc[i] += t[i];
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= nv) continue;
        if (bias) acc[i] += *(const fv*)(bias + E * c);
        if (RES == 1) acc[i] += ((const fv*)res)[row0 + c];
        if (RES == 2) {
            const bv b = ((const bv*)res)[row0 + c];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[i][e] += (float)b[e];
        }
        if (Z && OUT_BF16) {
            bv o;
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = (__bf16)acc[i][e];
            __builtin_nontemporal_store(o, (bv*)Z + row0 + c);
        } else if (Z) {
            __builtin_nontemporal_store(acc[i], (fv*)Z + row0 + c);
        }
        if (LN) {
            float u = (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
            if constexpr (E == 8) u += (acc[i][4] + acc[i][5]) + (acc[i][6] + acc[i][7]);
            sum += u;
        }
    }
    if (!LN) return;
    // LayerNorm of the summed row (f32 statistics, population variance,
    // two exact passes over the registers)
    const float mean = block_sum(sum, red) / (float)h;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
        if (threadIdx.x + 256 * i < nv)
#pragma unroll
            for (int e = 0; e < E; ++e) { const float d = acc[i][e] - mean; q += d * d; }
    const float inv = rsqrtf(block_sum(q, red) / (float)h + eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c >= nv) continue;
        bv o;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float v = (acc[i][e] - mean) * inv;
            if (gamma) v *= gamma[E * c + e];
            if (beta) v += beta[E * c + e];
            o[e] = (__bf16)v;
        }
        __builtin_nontemporal_store(o, (bv*)y + row0 + c);
    }
}

template <bool PB, bool RB, bool OB>
void launch_ps(void* Z, const void* parts, int P, int64_t n4, int h, const float* bias,
               const void* res, hipStream_t stream) {
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    hipLaunchKernelGGL((partial_sum_kernel<PB, RB, OB>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, Z, parts, P, n4, h, bias, res);
}

}  // namespace

hipError_t layernorm(const void* x, bool x_bf16, void* y, const float* gamma,
                     const float* beta, float eps, int64_t M, int64_t h, hipStream_t stream)
{
    // rows that fit the registers of one workgroup: the row-sum kernel with no
    // partials, x as the "residual" and only the normalised row written
    if (h % 4 == 0 && h <= 16384)
        return row_sum(nullptr, false, nullptr, false, 0, M, h, nullptr, x, x_bf16, y, gamma,
                       beta, eps, stream);
    const size_t lds = (size_t)h * sizeof(float);
    if (x_bf16)
        hipLaunchKernelGGL((layernorm_kernel<true>), dim3((unsigned)M), dim3(256), lds, stream,
                           x, (__bf16*)y, gamma, beta, eps, (int)h);
    else
        hipLaunchKernelGGL((layernorm_kernel<false>), dim3((unsigned)M), dim3(256), lds, stream,
                           x, (__bf16*)y, gamma, beta, eps, (int)h);
    return hipGetLastError();
}

hipError_t partial_sum(void* Z, bool out_bf16, const void* parts, bool parts_bf16, int P,
                       int64_t M, int64_t h, const float* bias,
                       const void* residual, bool res_bf16, hipStream_t stream)
{
    const int64_t n4 = M * h / 4;
    const int hh = (int)h;
#define TP_PS(PB, RB, OB) launch_ps<PB, RB, OB>(Z, parts, P, n4, hh, bias, residual, stream)
    if (parts_bf16) {
        if (res_bf16) { if (out_bf16) TP_PS(true, true, true); else TP_PS(true, true, false); }
        else          { if (out_bf16) TP_PS(true, false, true); else TP_PS(true, false, false); }
    } else {
        if (res_bf16) { if (out_bf16) TP_PS(false, true, true); else TP_PS(false, true, false); }
        else          { if (out_bf16) TP_PS(false, false, true); else TP_PS(false, false, false); }
    }
#undef TP_PS
    return hipGetLastError();
}

hipError_t row_sum(void* Z, bool out_bf16, const void* parts, bool parts_bf16, int P,
                   int64_t M, int64_t h, const float* bias, const void* residual, bool res_bf16,
                   void* ln_out, const float* gamma, const float* beta, float eps,
                   hipStream_t stream)
{
    // 8-element units when no f32 partial is read (16-byte bf16 loads), else 4
    const bool e8 = (P == 0 || parts_bf16) && h % 8 == 0;
    const int res = residual ? (res_bf16 ? 2 : 1) : 0;
    const dim3 grid((unsigned)M), block(256);
    __bf16* y = (__bf16*)ln_out;
#define TP_RS(PB, R, OB, L)                                                                    \
    do {                                                                                       \
        if (e8)                                                                                \
            hipLaunchKernelGGL((row_sum_kernel<PB, R, OB, L, 8>), grid, block, 0, stream, Z,   \
                               parts, P, M * h / 8, (int)h, bias, residual, y, gamma, beta,    \
                               eps);                                                           \
        else                                                                                   \
            hipLaunchKernelGGL((row_sum_kernel<PB, R, OB, L, 4>), grid, block, 0, stream, Z,   \
                               parts, P, M * h / 4, (int)h, bias, residual, y, gamma, beta,    \
                               eps);                                                           \
    } while (0)
#define TP_RS_RES(PB, OB, L) { if (res == 0) TP_RS(PB, 0, OB, L); \
        else if (res == 1) TP_RS(PB, 1, OB, L); else TP_RS(PB, 2, OB, L); }
    if (ln_out) {
        if (parts_bf16) { if (out_bf16) TP_RS_RES(true, true, true) else TP_RS_RES(true, false, true) }
        else            { if (out_bf16) TP_RS_RES(false, true, true) else TP_RS_RES(false, false, true) }
    } else {
        if (parts_bf16) { if (out_bf16) TP_RS_RES(true, true, false) else TP_RS_RES(true, false, false) }
        else            { if (out_bf16) TP_RS_RES(false, true, false) else TP_RS_RES(false, false, false) }
    }
#undef TP_RS_RES
#undef TP_RS
    return hipGetLastError();
}

}  // namespace tpk
