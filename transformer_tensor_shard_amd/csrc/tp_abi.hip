// extern "C" entry points of libtp.so (declared and documented in tp.h).
//
// Every entry point validates all of its arguments before enqueueing any work
// and returns a tp_status; the kernels themselves live in gemm_bf16.hip,
// gemm_f32.hip, attention.hip and norm_sum.hip.
#include "tp.h"
#include "tp_kernels.h"

#include <stdint.h>

#include <mutex>

#define TP_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kAlign = 256;            // workspace sub-buffer alignment
constexpr int64_t kHeadDim = 128;          // the attention kernel's head tile
constexpr int64_t kMaxLnWidth = 16384;     // the block's row kernels keep a row in registers
constexpr int64_t kMaxLnWidthWide = 32768; // tp_layernorm's wide-row kernel keeps it in LDS
constexpr int64_t kI32 = 0x7fffffffLL;
constexpr int kMaxGroup = 16;             // products per tp_matmul_grouped call

inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool is_dtype(int t) { return t == TP_F32 || t == TP_BF16; }
inline int64_t esize(int t) { return t == TP_BF16 ? 2 : 4; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline tp_status launched(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_LAUNCH; }

// The bf16 GEMM addresses a 256-row tile of an operand with 32-bit byte
// offsets and uses 32-bit tile counters.
bool gemm_bf16_fits(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M <= kI32 && N <= kI32 && K <= kI32 && lda * 2 * 256 < kI32 && ldb * 2 * 64 < kI32 &&
           ((M + 255) / 256) * ((N + 255) / 256) <= kI32;
}

tp_status check_linear(const void* X, int64_t ldx, const void* W, int64_t ldw, const void* bias,
                       const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int in,
                       int out, int epi) {
    if (!X || !W || !C) return TP_ERR_NULL;
    if (!is_dtype(in) || !is_dtype(out) || (epi != TP_EPI_NONE && epi != TP_EPI_GELU))
        return TP_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || ldx < K || ldw < N || ldc < N) return TP_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(W) || !aligned16(C) || (bias && !aligned16(bias)))
        return TP_ERR_ALIGN;
    if (in == TP_BF16) {
        if (K % 8 || N % 8 || ldx % 8 || ldw % 8 || ldc % 8 || !gemm_bf16_fits(M, N, K, ldx, ldw))
            return TP_ERR_SHAPE;
    } else if (M > kI32 || N > kI32 || K > kI32) {
        return TP_ERR_SHAPE;
    }
    return TP_OK;
}

hipError_t run_linear(const void* X, int64_t ldx, const void* W, int64_t ldw, const void* bias,
                      void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int in, int out,
                      bool gelu, hipStream_t st) {
    if (in == TP_BF16)
        return tpk::gemm_bf16(X, ldx, W, ldw, (const float*)bias, C, ldc, M, N, K,
                              out == TP_BF16, gelu, st);
    return tpk::gemm_f32((const float*)X, ldx, (const float*)W, ldw, (const float*)bias, C, ldc,
                         M, N, K, out == TP_BF16, gelu, st);
}

// ---- general bf16 product (tp_matmul) -------------------------------------
// A K-contiguous operand tile spans 256 rows of the operand, an M/N-contiguous
// one 64 K rows; the kernel addresses a tile with 32-bit byte offsets.
bool operand_fits(int64_t ld, bool k_contiguous) {
    return ld * 2 * (k_contiguous ? 256 : 64) < kI32;
}

int gemm_epi(int epi) {
    switch (epi) {
    case TP_EPI_GELU: return tpk::EPI_GELU;
    case TP_EPI_GELU_BWD: return tpk::EPI_GELU_BWD;
    case TP_EPI_GELU_SAVE: return tpk::EPI_DUAL;
    default: return tpk::EPI_NONE;
    }
}

bool matmul_supported(int ta, int tb, int out, int epi) {
    if (ta == 0 && tb == 0)
        return epi == TP_EPI_NONE || epi == TP_EPI_GELU || (epi == TP_EPI_GELU_SAVE && out == TP_BF16);
    if (ta == 0 && tb == 1) return epi == TP_EPI_NONE || epi == TP_EPI_GELU_BWD;
    if (ta == 1 && tb == 0) return epi == TP_EPI_NONE;
    return false;
}

tp_status check_matmul(const void* A, int64_t lda, int ta, const void* B, int64_t ldb, int tb,
                       const void* bias, const void* C, int64_t ldc, const void* aux,
                       int64_t ldaux, int64_t M, int64_t N, int64_t K, int out, int epi) {
    if (!A || !B || !C) return TP_ERR_NULL;
    if (!is_dtype(out) || !matmul_supported(ta, tb, out, epi)) return TP_ERR_DTYPE;
    const bool uses_aux = epi == TP_EPI_GELU_BWD || epi == TP_EPI_GELU_SAVE;
    if (uses_aux && !aux) return TP_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0 || M > kI32 || N > kI32 || K > kI32) return TP_ERR_SHAPE;
    if (lda < (ta ? M : K) || ldb < (tb ? K : N) || ldc < N || (uses_aux && ldaux < N))
        return TP_ERR_SHAPE;
    // every contiguous dimension and leading dimension a multiple of 8
    if ((ta ? M : K) % 8 || (tb ? K : N) % 8 || N % 8 || lda % 8 || ldb % 8 || ldc % 8 ||
        (uses_aux && ldaux % 8))
        return TP_ERR_SHAPE;
    // the GeLU-backward epilogue reads a tile's 256 rows of aux with 32-bit
    // byte offsets, as the K-contiguous operands are read
    if (!operand_fits(lda, !ta) || !operand_fits(ldb, tb != 0) ||
        (epi == TP_EPI_GELU_BWD && !operand_fits(ldaux, true)) ||
        ((M + 255) / 256) * ((N + 255) / 256) > kI32 / 8)
        return TP_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C) || (bias && !aligned16(bias)) ||
        (uses_aux && !aligned16(aux)))
        return TP_ERR_ALIGN;
    return TP_OK;
}

hipError_t run_matmul(const void* A, int64_t lda, int ta, const void* B, int64_t ldb, int tb,
                      const void* bias, void* C, int64_t ldc, void* aux, int64_t ldaux,
                      int64_t M, int64_t N, int64_t K, int out, int epi, hipStream_t st) {
    tpk::GemmBatch gb = {};
    gb.A[0] = (const __bf16*)A;
    gb.B[0] = (const __bf16*)B;
    gb.bias[0] = (const float*)bias;
    gb.C[0] = C;
    gb.aux[0] = (__bf16*)aux;
    gb.count = 1;
    const int layout = ta ? tpk::GEMM_TN : (tb ? tpk::GEMM_NT : tpk::GEMM_NN);
    return tpk::gemm_bf16_batched(gb, layout, gemm_epi(epi), lda, ldb, ldc, ldaux, M, N, K,
                                  out == TP_BF16, st);
}

// `n` bf16 products of one layout, output type and K but their own shapes in
// one grouped launch (no epilogue); the caller has validated every group.
// `spare` (spare_bytes, or NULL) is device memory free for the launch, which
// may then split its last wave of workgroups over K (f32 output).
struct Product {
    const void* A; int64_t lda; const void* B; int64_t ldb; void* C; int64_t ldc;
    int64_t M, N;
};
hipError_t run_grouped(const Product* p, int n, int64_t K, int ta, int tb, int out,
                       hipStream_t st, void* spare = nullptr, int64_t spare_bytes = 0) {
    tpk::GemmBatch gb = {};
    gb.count = n;
    gb.split_ws = (float*)spare;
    gb.split_ws_bytes = spare ? spare_bytes : 0;
    for (int i = 0; i < n; ++i) {
        gb.A[i] = (const __bf16*)p[i].A;
        gb.B[i] = (const __bf16*)p[i].B;
        gb.C[i] = p[i].C;
        gb.M[i] = (int)p[i].M;
        gb.N[i] = (int)p[i].N;
        gb.lda[i] = p[i].lda;
        gb.ldb[i] = p[i].ldb;
        gb.ldc[i] = p[i].ldc;
    }
    const int layout = ta ? tpk::GEMM_TN : (tb ? tpk::GEMM_NT : tpk::GEMM_NN);
    return tpk::gemm_bf16_grouped(gb, layout, tpk::EPI_NONE, 0, K, out == TP_BF16, st);
}

// ---- MLP shard ------------------------------------------------------------
int64_t mlp_ws(int64_t M, int64_t f, int in) { return align_up(M * f * esize(in)); }

tp_status check_mlp(const void* X, const void* A_i, const void* a_i, const void* B_i,
                    const void* Z_i, int64_t M, int64_t h, int64_t f, int in, int out) {
    if (!X || !A_i || !B_i || !Z_i) return TP_ERR_NULL;
    if (!is_dtype(in) || !is_dtype(out)) return TP_ERR_DTYPE;
    if (M <= 0 || h <= 0 || f <= 0) return TP_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Z_i) ||
        (a_i && !aligned16(a_i)))
        return TP_ERR_ALIGN;
    if (in == TP_BF16 && (h % 8 || f % 8 || !gemm_bf16_fits(M, f, h, h, f) ||
                          !gemm_bf16_fits(M, h, f, f, h)))
        return TP_ERR_SHAPE;
    if (in == TP_F32 && (M > kI32 || h > kI32 || f > kI32)) return TP_ERR_SHAPE;
    return TP_OK;
}

hipError_t run_mlp(const void* X, const void* A_i, const void* a_i, const void* B_i, void* Z_i,
                   void* ws, int64_t M, int64_t h, int64_t f, int in, int out, hipStream_t st) {
    // Y'_i = GeLU(X·A_i + a_i), kept in the input precision (column-parallel, §2.1)
    hipError_t e = run_linear(X, h, A_i, f, a_i, ws, f, M, f, h, in, in, true, st);
    if (e != hipSuccess) return e;
    // Z_i = Y'_i·B_i, the rank's partial sum (row-parallel, §2.1)
    return run_linear(ws, f, B_i, h, nullptr, Z_i, h, M, h, f, in, out, false, st);
}

// ---- attention shard ------------------------------------------------------
struct AttnWs { int64_t qkv, o, total; };
AttnWs attn_ws(int64_t b, int64_t s, int64_t H_l, int64_t d) {
    const int64_t M = b * s;
    AttnWs w;
    w.qkv = 0;
    w.o = align_up(M * 3 * H_l * d * 2);
    w.total = w.o + align_up(M * H_l * d * 2);
    return w;
}

tp_status check_attn_shape(int64_t b, int64_t s, int64_t h, int64_t H_l, int64_t d) {
    if (b <= 0 || s <= 0 || h <= 0 || H_l <= 0 || d <= 0) return TP_ERR_SHAPE;
    if (d != kHeadDim || h % 8) return TP_ERR_SHAPE;
    const int64_t M = b * s, n3 = 3 * H_l * d;
    if (!gemm_bf16_fits(M, n3, h, h, n3) || !gemm_bf16_fits(M, h, H_l * d, H_l * d, h))
        return TP_ERR_SHAPE;
    // the attention kernel addresses one sequence of qkv with 32-bit offsets
    if (s * n3 * 2 >= kI32 || ((s + 127) / 128) * (b * H_l + 7) > kI32) return TP_ERR_SHAPE;
    return TP_OK;
}

hipError_t run_attn(const void* X, const void* Wqkv, const void* Wo, void* Z, void* ws,
                    int64_t b, int64_t s, int64_t h, int64_t H_l, int64_t d, bool causal, int out,
                    hipStream_t st) {
    const int64_t M = b * s, n3 = 3 * H_l * d;
    const AttnWs w = attn_ws(b, s, H_l, d);
    char* qkv = (char*)ws + w.qkv;
    char* O = (char*)ws + w.o;
    // [Q|K|V] = X·W_qkv_i for the local heads (column-parallel, §3.2)
    hipError_t e = tpk::gemm_bf16(X, h, Wqkv, n3, nullptr, qkv, n3, M, n3, h, true, false, st);
    if (e != hipSuccess) return e;
    e = tpk::attention_fwd(qkv, n3, O, b, s, H_l, causal, st);
    if (e != hipSuccess) return e;
    // Z_i = O_i·W_o_i (row-parallel partial, §3.2)
    return tpk::gemm_bf16(O, H_l * d, Wo, h, nullptr, Z, h, M, h, H_l * d, out == TP_BF16, false, st);
}

// ---- block ----------------------------------------------------------------
// The P emulated ranks' products have identical shapes, so each step of the
// block runs as one grouped launch over all ranks (each tile still belongs to
// one rank and uses only that rank's slice); every rank keeps its own
// projections, attention output, activations and f32 partial in the
// workspace, sized for HBM rather than folded early.
struct BlockWs { int64_t xn, parts, x1, qkv, o, y, total; };
BlockWs block_ws(int64_t b, int64_t s, int64_t h, int64_t H, int64_t d, int64_t F, int P) {
    const int64_t M = b * s, Hl = H / P, f = F / P;
    BlockWs w;
    w.xn = 0;
    w.parts = align_up(M * h * 2);
    w.x1 = w.parts + align_up((int64_t)P * M * h * 4);
    const int64_t scratch = w.x1 + align_up(M * h * 4);
    // attention scratch (all ranks' Q|K|V and O) and the MLP scratch (all
    // ranks' GeLU(X·A_r)) are never live at the same time
    w.qkv = scratch;
    w.o = w.qkv + align_up((int64_t)P * M * 3 * Hl * d * 2);
    w.y = scratch;
    const int64_t attn_end = w.o + align_up((int64_t)P * M * Hl * d * 2);
    const int64_t mlp_end = w.y + align_up((int64_t)P * M * f * 2);
    w.total = attn_end > mlp_end ? attn_end : mlp_end;
    return w;
}

// C[r] = epi(A[r]·B[r]) for ranks r0 .. r0+n-1 in launches of up to kMaxBatch
template <typename FA, typename FB, typename FC>
hipError_t grouped(int P, FA a_of, FB b_of, FC c_of, int64_t lda, int64_t ldb, int64_t ldc,
                   int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu, hipStream_t st) {
    for (int r0 = 0; r0 < P; r0 += tpk::kMaxBatch) {
        tpk::GemmBatch gb = {};
        gb.count = P - r0 < tpk::kMaxBatch ? P - r0 : tpk::kMaxBatch;
        for (int i = 0; i < gb.count; ++i) {
            gb.A[i] = (const __bf16*)a_of(r0 + i);
            gb.B[i] = (const __bf16*)b_of(r0 + i);
            gb.C[i] = c_of(r0 + i);
        }
        const hipError_t e = tpk::gemm_bf16_batched(gb, lda, ldb, ldc, M, N, K, out_bf16, gelu, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

// ===========================================================================
TP_EXPORT const char* tp_status_string(int status) {
    switch (status) {
        case TP_OK: return "ok";
        case TP_ERR_NULL: return "a required pointer is NULL";
        case TP_ERR_SHAPE: return "unsupported or inconsistent shape";
        case TP_ERR_DTYPE: return "unsupported dtype or epilogue code";
        case TP_ERR_ALIGN: return "pointer not 16-byte aligned";
        case TP_ERR_WORKSPACE: return "workspace missing or too small";
        case TP_ERR_LAUNCH: return "kernel launch failed";
        case TP_ERR_SCRATCH: return "size exceeds the fixed scratch of an allocation-free call";
        default: return "unknown status";
    }
}

TP_EXPORT int tp_abi_version(void) { return 2; }

TP_EXPORT tp_status tp_linear(const void* X, int64_t ldx, const void* W, int64_t ldw,
                              const void* bias, void* C, int64_t ldc, int64_t M, int64_t N,
                              int64_t K, int in, int out, int epilogue, void* stream) {
    const tp_status s = check_linear(X, ldx, W, ldw, bias, C, ldc, M, N, K, in, out, epilogue);
    if (s != TP_OK) return s;
    return launched(run_linear(X, ldx, W, ldw, bias, C, ldc, M, N, K, in, out,
                               epilogue == TP_EPI_GELU, as_stream(stream)));
}

TP_EXPORT tp_status tp_linear_batched(const void* const* X, int64_t ldx, const void* const* W,
                                      int64_t ldw, const void* const* bias, void* const* C,
                                      int64_t ldc, int count, int64_t M, int64_t N, int64_t K,
                                      int in, int out, int epilogue, void* stream) {
    if (!X || !W || !C) return TP_ERR_NULL;
    if (count <= 0) return TP_ERR_SHAPE;
    for (int g = 0; g < count; ++g) {
        const tp_status s = check_linear(X[g], ldx, W[g], ldw, bias ? bias[g] : nullptr, C[g], ldc,
                                         M, N, K, in, out, epilogue);
        if (s != TP_OK) return s;
    }
    const hipStream_t st = as_stream(stream);
    const bool gelu = epilogue == TP_EPI_GELU;
    if (in != TP_BF16) {
        for (int g = 0; g < count; ++g) {
            const hipError_t e = run_linear(X[g], ldx, W[g], ldw, bias ? bias[g] : nullptr, C[g],
                                            ldc, M, N, K, in, out, gelu, st);
            if (e != hipSuccess) return TP_ERR_LAUNCH;
        }
        return TP_OK;
    }
    for (int g0 = 0; g0 < count; g0 += tpk::kMaxBatch) {
        tpk::GemmBatch gb = {};
        gb.count = count - g0 < tpk::kMaxBatch ? count - g0 : tpk::kMaxBatch;
        for (int i = 0; i < gb.count; ++i) {
            gb.A[i] = (const __bf16*)X[g0 + i];
            gb.B[i] = (const __bf16*)W[g0 + i];
            gb.bias[i] = bias ? (const float*)bias[g0 + i] : nullptr;
            gb.C[i] = C[g0 + i];
        }
        if (tpk::gemm_bf16_batched(gb, ldx, ldw, ldc, M, N, K, out == TP_BF16, gelu, st))
            return TP_ERR_LAUNCH;
    }
    return TP_OK;
}

TP_EXPORT size_t tp_mlp_shard_workspace(int64_t M, int64_t f, int in) {
    if (M <= 0 || f <= 0 || !is_dtype(in)) return 0;
    return (size_t)mlp_ws(M, f, in);
}

TP_EXPORT tp_status tp_mlp_shard(const void* X, const void* A_i, const void* a_i,
                                 const void* B_i, void* Z_i, void* ws, size_t ws_bytes,
                                 int64_t M, int64_t h, int64_t f, int in, int out, void* stream) {
    tp_status s = check_mlp(X, A_i, a_i, B_i, Z_i, M, h, f, in, out);
    if (s != TP_OK) return s;
    if (!ws || ws_bytes < (size_t)mlp_ws(M, f, in)) return TP_ERR_WORKSPACE;
    if (!aligned16(ws)) return TP_ERR_ALIGN;
    return launched(run_mlp(X, A_i, a_i, B_i, Z_i, ws, M, h, f, in, out, as_stream(stream)));
}

// ---- allocation-free MLP share ---------------------------------------------
// The scratch of tp_mlp_shard_noalloc: a fixed device array that every GPU the
// library runs on holds until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host the name is only a stand-in); it
// looks up each device's address once with hipGetSymbolAddress and passes
// that.
constexpr int64_t kNoAllocScratchBytes = 64ll << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the device that `stream` runs on (looked up
// with that device current, once per device).
hipError_t scratch_on_device(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    hipDevice_t dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Token rows of Y'_i that fit the scratch at width f: a multiple of 256 (the
// GEMM's tile height), 0 when not even one tile row fits.
int64_t noalloc_rows(int64_t f, int in) {
    return (kNoAllocScratchBytes / (f * esize(in))) / 256 * 256;
}
}  // namespace

TP_EXPORT tp_status tp_mlp_shard_noalloc(const void* X, const void* A_i, const void* a_i,
                                         const void* B_i, void* Z_i, int64_t M, int64_t h,
                                         int64_t f, int in, int out, void* stream) {
    tp_status s = check_mlp(X, A_i, a_i, B_i, Z_i, M, h, f, in, out);
    if (s != TP_OK) return s;
    const int64_t rows = noalloc_rows(f, in);
    if (rows < 256) return TP_ERR_SCRATCH;
    hipStream_t st = as_stream(stream);
    void* ws = nullptr;
    if (scratch_on_device(st, &ws) != hipSuccess) return TP_ERR_LAUNCH;
    // Token rows are independent: the share runs on row blocks whose Y'_i fits
    // the scratch, each with the kernels (and the per-element summation order)
    // of tp_mlp_shard, so the result is the same bit for bit.
    for (int64_t m0 = 0; m0 < M; m0 += rows) {
        const int64_t mc = M - m0 < rows ? M - m0 : rows;
        const hipError_t e = run_mlp((const char*)X + m0 * h * esize(in), A_i, a_i, B_i,
                                     (char*)Z_i + m0 * h * esize(out), ws, mc, h, f, in, out, st);
        if (e != hipSuccess) return TP_ERR_LAUNCH;
    }
    return TP_OK;
}

TP_EXPORT tp_status tp_matmul(const void* A, int64_t lda, int trans_a, const void* B,
                              int64_t ldb, int trans_b, const void* bias, void* C, int64_t ldc,
                              void* aux, int64_t ldaux, int64_t M, int64_t N, int64_t K, int out,
                              int epilogue, void* stream) {
    const tp_status s = check_matmul(A, lda, trans_a, B, ldb, trans_b, bias, C, ldc, aux, ldaux,
                                     M, N, K, out, epilogue);
    if (s != TP_OK) return s;
    return launched(run_matmul(A, lda, trans_a, B, ldb, trans_b, bias, C, ldc, aux, ldaux, M, N,
                               K, out, epilogue, as_stream(stream)));
}

TP_EXPORT tp_status tp_matmul_grouped(const void* const* A, const int64_t* lda, int trans_a,
                                      const void* const* B, const int64_t* ldb, int trans_b,
                                      void* const* C, const int64_t* ldc, const int64_t* M,
                                      const int64_t* N, int count, int64_t K, int out,
                                      void* ws, size_t ws_bytes, void* stream) {
    if (!A || !lda || !B || !ldb || !C || !ldc || !M || !N) return TP_ERR_NULL;
    if (count <= 0 || count > kMaxGroup) return TP_ERR_SHAPE;
    if (ws && !aligned16(ws)) return TP_ERR_ALIGN;
    Product p[kMaxGroup];
    for (int g = 0; g < count; ++g) {
        const tp_status s = check_matmul(A[g], lda[g], trans_a, B[g], ldb[g], trans_b, nullptr,
                                         C[g], ldc[g], nullptr, 0, M[g], N[g], K, out,
                                         TP_EPI_NONE);
        if (s != TP_OK) return s;
        p[g] = {A[g], lda[g], B[g], ldb[g], C[g], ldc[g], M[g], N[g]};
    }
    const int64_t spare = ws_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)ws_bytes;
    return launched(run_grouped(p, count, K, trans_a, trans_b, out, as_stream(stream), ws, spare));
}

TP_EXPORT int tp_gemm_tile_cols(int trans_a, int trans_b, int epilogue, int count,
                                const int64_t* M, const int64_t* N, int64_t K) {
    if (!M || !N || count <= 0 || count > kMaxGroup || K <= 0) return 0;
    if ((trans_a && trans_b) || epilogue < TP_EPI_NONE || epilogue > TP_EPI_GELU_SAVE) return 0;
    tpk::GemmBatch gb = {};
    gb.count = count;
    for (int g = 0; g < count; ++g) {
        if (M[g] <= 0 || N[g] <= 0 || M[g] >= kI32 || N[g] >= kI32) return 0;
        gb.M[g] = (int)M[g];
        gb.N[g] = (int)N[g];
    }
    const int layout = trans_a ? tpk::GEMM_TN : (trans_b ? tpk::GEMM_NT : tpk::GEMM_NN);
    return tpk::gemm_tile_cols(gb, layout, gemm_epi(epilogue), K);
}

// ---- MLP shard: training forward and backward ------------------------------
namespace {
struct MlpBwdWs {
    int64_t dy, part, total;   // byte offsets: dY bf16 [M,f]; bias partials f32 [chunks,f]
};
MlpBwdWs mlp_bwd_ws(int64_t M, int64_t f) {
    MlpBwdWs w;
    w.dy = 0;
    w.part = align_up(M * f * 2);
    w.total = w.part + align_up(tpk::col_sum_chunks(M) * f * 4);
    return w;
}

tp_status check_mlp_train(int64_t M, int64_t h, int64_t f) {
    if (M <= 0 || h <= 0 || f <= 0 || M > kI32 || h > kI32 || f > kI32) return TP_ERR_SHAPE;
    if (h % 8 || f % 8) return TP_ERR_SHAPE;
    // K-contiguous operands have leading dimension h or f, M/N-contiguous ones too
    if (!operand_fits(h, true) || !operand_fits(f, true)) return TP_ERR_SHAPE;
    const int64_t big = M > h ? (M > f ? M : f) : (h > f ? h : f);
    if (((big + 255) / 256) * ((big + 255) / 256) > kI32 / 8) return TP_ERR_SHAPE;
    if (tpk::col_sum_chunks(M) > 65535) return TP_ERR_SHAPE;
    return TP_OK;
}
}  // namespace

TP_EXPORT tp_status tp_mlp_shard_train_fwd(const void* X, const void* A_i, const void* a_i,
                                           const void* B_i, void* Z_i, void* Y_i, void* Yp_i,
                                           int64_t M, int64_t h, int64_t f, int out,
                                           void* stream) {
    if (!X || !A_i || !B_i || !Z_i || !Y_i || !Yp_i) return TP_ERR_NULL;
    if (!is_dtype(out)) return TP_ERR_DTYPE;
    tp_status s = check_mlp_train(M, h, f);
    if (s != TP_OK) return s;
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Z_i) ||
        !aligned16(Y_i) || !aligned16(Yp_i) || (a_i && !aligned16(a_i)))
        return TP_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    // Y = X·A_i + a_i and Y' = GeLU(Y) in one epilogue; then Z_i = Y'·B_i
    if (run_matmul(X, h, 0, A_i, f, 0, a_i, Yp_i, f, Y_i, f, M, f, h, TP_BF16,
                   TP_EPI_GELU_SAVE, st))
        return TP_ERR_LAUNCH;
    return launched(run_matmul(Yp_i, f, 0, B_i, h, 0, nullptr, Z_i, h, nullptr, 0, M, h, f, out,
                               TP_EPI_NONE, st));
}

TP_EXPORT size_t tp_mlp_shard_backward_workspace(int64_t M, int64_t f) {
    if (M <= 0 || f <= 0) return 0;
    return (size_t)mlp_bwd_ws(M, f).total;
}

TP_EXPORT tp_status tp_mlp_shard_backward(const void* X, const void* A_i, const void* B_i,
                                          const void* Y_i, const void* Yp_i, const void* dZ,
                                          void* dX_i, void* dA_i, void* dB_i, void* da_i,
                                          void* ws, size_t ws_bytes, int64_t M, int64_t h,
                                          int64_t f, int dx_dtype, void* stream) {
    if (!X || !A_i || !B_i || !Y_i || !Yp_i || !dZ || !dX_i || !dA_i || !dB_i)
        return TP_ERR_NULL;
    if (!is_dtype(dx_dtype)) return TP_ERR_DTYPE;
    tp_status s = check_mlp_train(M, h, f);
    if (s != TP_OK) return s;
    const MlpBwdWs w = mlp_bwd_ws(M, f);
    if (!ws || ws_bytes < (size_t)w.total) return TP_ERR_WORKSPACE;
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Y_i) ||
        !aligned16(Yp_i) || !aligned16(dZ) || !aligned16(dX_i) || !aligned16(dA_i) ||
        !aligned16(dB_i) || (da_i && !aligned16(da_i)) || !aligned16(ws))
        return TP_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    char* base = (char*)ws;
    void* dY = base + w.dy;
    // dY = (dZ·B_i^T) ⊙ GeLU'(Y_i)            [M,f] bf16
    if (run_matmul(dZ, h, 0, B_i, h, 1, nullptr, dY, f, (void*)Y_i, f, M, f, h, TP_BF16,
                   TP_EPI_GELU_BWD, st))
        return TP_ERR_LAUNCH;
    // dB_i = Y'_i^T·dZ [f,h] and dA_i = X^T·dY [h,f], f32, in one grouped
    // launch: each alone leaves a partly filled last wave of tiles
    const Product wgrad[2] = {{Yp_i, f, dZ, h, dB_i, h, f, h}, {X, h, dY, f, dA_i, f, h, f}};
    if (run_grouped(wgrad, 2, M, 1, 0, TP_F32, st)) return TP_ERR_LAUNCH;
    // dX_i = dY·A_i^T                          [M,h] partial over ranks
    if (run_matmul(dY, f, 0, A_i, f, 1, nullptr, dX_i, h, nullptr, 0, M, h, f, dx_dtype,
                   TP_EPI_NONE, st))
        return TP_ERR_LAUNCH;
    if (da_i)
        return launched(tpk::col_sum((float*)da_i, dY, f, M, f, (float*)(base + w.part), st));
    return TP_OK;
}

TP_EXPORT size_t tp_attn_shard_workspace(int64_t b, int64_t s, int64_t H_l, int64_t d) {
    if (b <= 0 || s <= 0 || H_l <= 0 || d <= 0) return 0;
    return (size_t)attn_ws(b, s, H_l, d).total;
}

TP_EXPORT tp_status tp_attn_shard(const void* X, const void* W_qkv_i, const void* W_o_i,
                                  void* Z_i, void* ws, size_t ws_bytes, int64_t b, int64_t s,
                                  int64_t h, int64_t H_l, int64_t d, int causal, int out,
                                  void* stream) {
    if (!X || !W_qkv_i || !W_o_i || !Z_i) return TP_ERR_NULL;
    if (!is_dtype(out)) return TP_ERR_DTYPE;
    tp_status st = check_attn_shape(b, s, h, H_l, d);
    if (st != TP_OK) return st;
    if (!aligned16(X) || !aligned16(W_qkv_i) || !aligned16(W_o_i) || !aligned16(Z_i))
        return TP_ERR_ALIGN;
    if (!ws || ws_bytes < (size_t)attn_ws(b, s, H_l, d).total) return TP_ERR_WORKSPACE;
    if (!aligned16(ws)) return TP_ERR_ALIGN;
    return launched(run_attn(X, W_qkv_i, W_o_i, Z_i, ws, b, s, h, H_l, d, causal != 0, out,
                             as_stream(stream)));
}

TP_EXPORT tp_status tp_attention_core(const void* qkv, int64_t ld_qkv, void* O, int64_t b,
                                      int64_t s, int64_t H_l, int64_t d, int causal,
                                      void* stream) {
    if (!qkv || !O) return TP_ERR_NULL;
    if (b <= 0 || s <= 0 || H_l <= 0 || d != kHeadDim || ld_qkv < 3 * H_l * d || ld_qkv % 8)
        return TP_ERR_SHAPE;
    if (s * ld_qkv * 2 >= kI32 || ((s + 127) / 128) * (b * H_l + 7) > kI32) return TP_ERR_SHAPE;
    if (!aligned16(qkv) || !aligned16(O)) return TP_ERR_ALIGN;
    return launched(tpk::attention_fwd(qkv, ld_qkv, O, b, s, H_l, causal != 0, as_stream(stream)));
}

// ---- attention with Q, K, V split along the feature dimension -------------
TP_EXPORT size_t tp_attention_kv_split_workspace(int64_t b, int64_t s, int64_t H, int64_t d,
                                                 int P) {
    if (b <= 0 || s <= 0 || H <= 0 || d <= 0 || P <= 0) return 0;
    return (size_t)tpk::kv_split_workspace_bytes(b * H, s, d, P);
}

TP_EXPORT tp_status tp_attention_kv_split(const void* qkv, int64_t ld_qkv, void* O, int64_t ldo,
                                          int64_t b, int64_t s, int64_t H, int64_t d, int P,
                                          int causal, void* ws, size_t ws_bytes, void* stream) {
    if (!qkv || !O) return TP_ERR_NULL;
    if (b <= 0 || s <= 0 || H <= 0 || d <= 0 || P <= 0 || d % P || (d / P) % 8 || s % 8 ||
        s > tpk::kKvMaxS || ld_qkv < 3 * H * d || ld_qkv % 8 || ldo < H * d || ldo % 8)
        return TP_ERR_SHAPE;
    if (s * ld_qkv * 2 >= kI32 || b * H > kI32 / s) return TP_ERR_SHAPE;
    if (!ws || ws_bytes < tp_attention_kv_split_workspace(b, s, H, d, P)) return TP_ERR_WORKSPACE;
    if (!aligned16(qkv) || !aligned16(O) || !aligned16(ws)) return TP_ERR_ALIGN;
    return launched(tpk::kv_split_attention((const __bf16*)qkv, ld_qkv, (__bf16*)O, ldo, (int)b,
                                            (int)s, (int)H, (int)d, P, causal != 0, ws,
                                            as_stream(stream)));
}

// ---- attention: training forward and backward ----------------------------
namespace {
tp_status check_core(int64_t ld_qkv, int64_t b, int64_t s, int64_t H_l, int64_t d) {
    if (b <= 0 || s <= 0 || H_l <= 0 || d != kHeadDim || ld_qkv < 3 * H_l * d || ld_qkv % 8)
        return TP_ERR_SHAPE;
    if (s * ld_qkv * 2 >= kI32 || ((s + 127) / 128) * (b * H_l + 7) > kI32) return TP_ERR_SHAPE;
    return TP_OK;
}

struct AttnBwdWs { int64_t dO, dqkv, D, total; };
AttnBwdWs attn_bwd_ws(int64_t b, int64_t s, int64_t H_l, int64_t d) {
    const int64_t M = b * s;
    AttnBwdWs w;
    w.dO = 0;
    w.dqkv = align_up(M * H_l * d * 2);
    w.D = w.dqkv + align_up(M * 3 * H_l * d * 2);
    w.total = w.D + align_up(M * H_l * 4);
    return w;
}
}  // namespace

TP_EXPORT tp_status tp_attention_core_train(const void* qkv, int64_t ld_qkv, void* O, float* lse,
                                            int64_t b, int64_t s, int64_t H_l, int64_t d,
                                            int causal, void* stream) {
    if (!qkv || !O || !lse) return TP_ERR_NULL;
    tp_status st = check_core(ld_qkv, b, s, H_l, d);
    if (st != TP_OK) return st;
    if (!aligned16(qkv) || !aligned16(O) || !aligned16(lse)) return TP_ERR_ALIGN;
    return launched(tpk::attention_fwd(qkv, ld_qkv, O, b, s, H_l, causal != 0, as_stream(stream),
                                       1, 0, 0, lse));
}

TP_EXPORT tp_status tp_attention_core_backward(const void* qkv, int64_t ld_qkv, const void* O,
                                               const void* dO, const float* lse, void* dqkv,
                                               float* D_ws, int64_t b, int64_t s, int64_t H_l,
                                               int64_t d, int causal, void* stream) {
    if (!qkv || !O || !dO || !lse || !dqkv || !D_ws) return TP_ERR_NULL;
    tp_status st = check_core(ld_qkv, b, s, H_l, d);
    if (st != TP_OK) return st;
    if (!aligned16(qkv) || !aligned16(O) || !aligned16(dO) || !aligned16(lse) ||
        !aligned16(dqkv) || !aligned16(D_ws))
        return TP_ERR_ALIGN;
    return launched(tpk::attention_bwd(qkv, ld_qkv, O, dO, lse, D_ws, dqkv, b, s, H_l,
                                       causal != 0, as_stream(stream)));
}

TP_EXPORT tp_status tp_attn_shard_train_fwd(const void* X, const void* W_qkv_i,
                                            const void* W_o_i, void* Z_i, void* qkv, void* O,
                                            float* lse, int64_t b, int64_t s, int64_t h,
                                            int64_t H_l, int64_t d, int causal, int out,
                                            void* stream) {
    if (!X || !W_qkv_i || !W_o_i || !Z_i || !qkv || !O || !lse) return TP_ERR_NULL;
    if (!is_dtype(out)) return TP_ERR_DTYPE;
    tp_status st = check_attn_shape(b, s, h, H_l, d);
    if (st != TP_OK) return st;
    const void* ptrs[] = {X, W_qkv_i, W_o_i, Z_i, qkv, O, lse};
    for (const void* p : ptrs)
        if (!aligned16(p)) return TP_ERR_ALIGN;
    const hipStream_t stm = as_stream(stream);
    const int64_t M = b * s, HD = H_l * d, n3 = 3 * HD;
    if (tpk::gemm_bf16(X, h, W_qkv_i, n3, nullptr, qkv, n3, M, n3, h, true, false, stm))
        return TP_ERR_LAUNCH;
    if (tpk::attention_fwd(qkv, n3, O, b, s, H_l, causal != 0, stm, 1, 0, 0, lse))
        return TP_ERR_LAUNCH;
    return launched(tpk::gemm_bf16(O, HD, W_o_i, h, nullptr, Z_i, h, M, h, HD, out == TP_BF16,
                                   false, stm));
}

TP_EXPORT size_t tp_attn_shard_backward_workspace(int64_t b, int64_t s, int64_t H_l, int64_t d) {
    if (b <= 0 || s <= 0 || H_l <= 0 || d <= 0) return 0;
    return (size_t)attn_bwd_ws(b, s, H_l, d).total;
}

TP_EXPORT tp_status tp_attn_shard_backward(const void* X, const void* W_qkv_i, const void* W_o_i,
                                           const void* qkv, const void* O, const float* lse,
                                           const void* dZ, void* dX_i, void* dW_qkv_i,
                                           void* dW_o_i, void* ws, size_t ws_bytes, int64_t b,
                                           int64_t s, int64_t h, int64_t H_l, int64_t d,
                                           int causal, int dx_dtype, void* stream) {
    if (!X || !W_qkv_i || !W_o_i || !qkv || !O || !lse || !dZ || !dX_i || !dW_qkv_i || !dW_o_i)
        return TP_ERR_NULL;
    if (!is_dtype(dx_dtype)) return TP_ERR_DTYPE;
    tp_status st = check_attn_shape(b, s, h, H_l, d);
    if (st != TP_OK) return st;
    const int64_t M = b * s, HD = H_l * d, n3 = 3 * HD;
    // the weight-gradient products read X, O and dqkv with the token as their row
    if (!operand_fits(h, false) || !operand_fits(n3, true) || !operand_fits(h, true))
        return TP_ERR_SHAPE;
    const AttnBwdWs w = attn_bwd_ws(b, s, H_l, d);
    if (!ws || ws_bytes < (size_t)w.total) return TP_ERR_WORKSPACE;
    const void* ptrs[] = {X, W_qkv_i, W_o_i, qkv, O, lse, dZ, dX_i, dW_qkv_i, dW_o_i, ws};
    for (const void* p : ptrs)
        if (!aligned16(p)) return TP_ERR_ALIGN;
    const hipStream_t stm = as_stream(stream);
    char* base = (char*)ws;
    void* dO = base + w.dO;
    void* dqkv = base + w.dqkv;
    float* Dv = (float*)(base + w.D);
    // dO = dZ·W_o,i^T                           [M, H_l·d] bf16
    if (run_matmul(dZ, h, 0, W_o_i, h, 1, nullptr, dO, HD, nullptr, 0, M, HD, h, TP_BF16,
                   TP_EPI_NONE, stm))
        return TP_ERR_LAUNCH;
    // dQ, dK, dV of the local heads            [M, 3·H_l·d] bf16
    if (tpk::attention_bwd(qkv, n3, O, dO, lse, Dv, dqkv, b, s, H_l, causal != 0, stm))
        return TP_ERR_LAUNCH;
    // dW_qkv,i = X^T·dqkv [h, 3·H_l·d] and dW_o,i = O^T·dZ [H_l·d, h], f32, in
    // one grouped launch (dW_o,i alone has too few tiles to fill the GPU);
    // dO is dead by now and its buffer serves a split of the launch's last
    // wave over K
    const Product wgrad[2] = {{X, h, dqkv, n3, dW_qkv_i, n3, h, n3},
                              {O, HD, dZ, h, dW_o_i, h, HD, h}};
    if (run_grouped(wgrad, 2, M, 1, 0, TP_F32, stm, dO, M * HD * 2)) return TP_ERR_LAUNCH;
    // dX_i = dqkv·W_qkv,i^T                      [M, h] partial over ranks
    return launched(run_matmul(dqkv, n3, 0, W_qkv_i, n3, 1, nullptr, dX_i, h, nullptr, 0, M, h,
                               n3, dx_dtype, TP_EPI_NONE, stm));
}

// ---- vocabulary ends: vocab-parallel embedding and cross-entropy -----------
namespace {
int64_t ce_ntn(int64_t V_r) { return (V_r + 127) / 128; }   // 128-column pieces per row
int64_t ce_tiles_bytes(int64_t M, int64_t V_r) { return align_up(M * ce_ntn(V_r) * 2 * 4); }
int64_t ce_stats_bytes(int64_t M) { return align_up(3 * M * 4); }

tp_status check_vocab(int64_t M, int64_t h, int64_t V_r) {
    if (M <= 0 || h <= 0 || V_r <= 0 || M > kI32 || h > kI32 || V_r > kI32) return TP_ERR_SHAPE;
    if (h % 8 || V_r % 8) return TP_ERR_SHAPE;
    return TP_OK;
}

// logits H·E_r^T of `count` ranks (one grouped NT launch) reduced to each
// rank's [3][M] statistics at stats + 3·M·g; tiles: [count][M][ntn][2] scratch
hipError_t run_ce_ranks(const void* H, const void* const* E, int count, const int* targets,
                        int64_t M, int64_t h, int64_t V_r, int64_t vstart0, float* stats,
                        float* tiles, hipStream_t st) {
    // each rank's logits rows leave statistics per 128-column piece (the same
    // values whichever output-tile width the GEMM takes)
    const int64_t ntn = ce_ntn(V_r);
    for (int g0 = 0; g0 < count; g0 += tpk::kMaxBatch) {
        const int n = count - g0 < tpk::kMaxBatch ? count - g0 : tpk::kMaxBatch;
        tpk::GemmBatch gb = {};
        gb.count = n;
        gb.targets = targets;
        for (int i = 0; i < n; ++i) {
            const int g = g0 + i;
            float* sg = stats + 3 * M * g;
            if (hipError_t e = tpk::fill_zero(sg + 2 * M, M, st)) return e;
            gb.A[i] = (const __bf16*)H;
            gb.B[i] = (const __bf16*)E[g];
            gb.C[i] = tiles + M * ntn * 2 * g;
            gb.aux[i] = (__bf16*)(sg + 2 * M);
            gb.vstart[i] = (int)(vstart0 + V_r * g);
        }
        if (hipError_t e = tpk::gemm_bf16_batched(gb, tpk::GEMM_NT, tpk::EPI_CE_STATS, h, h, 0, 0,
                                                  M, V_r, h, false, st))
            return e;
    }
    for (int g = 0; g < count; ++g)
        if (hipError_t e = tpk::ce_rank_reduce(tiles + M * ntn * 2 * g, (int)ntn, M,
                                               stats + 3 * M * g, st))
            return e;
    return hipSuccess;
}
}  // namespace

TP_EXPORT tp_status tp_vocab_embedding_shard(const int32_t* tokens, int64_t M, const void* E_r,
                                             int64_t V_r, int64_t h, int64_t vocab_start,
                                             void* out, int out_dtype, void* stream) {
    if (!tokens || !E_r || !out) return TP_ERR_NULL;
    if (!is_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (tp_status s = check_vocab(M, h, V_r)) return s;
    if (!aligned16(E_r) || !aligned16(out) || (reinterpret_cast<uintptr_t>(tokens) & 3))
        return TP_ERR_ALIGN;
    return launched(tpk::embed_shard(tokens, M, E_r, V_r, h, vocab_start, out,
                                     out_dtype == TP_BF16, as_stream(stream)));
}

TP_EXPORT size_t tp_vocab_ce_shard_workspace(int64_t M, int64_t V_r) {
    if (M <= 0 || V_r <= 0) return 0;
    return (size_t)ce_tiles_bytes(M, V_r);
}

TP_EXPORT tp_status tp_vocab_ce_shard(const void* H, const void* E_r, const int32_t* targets,
                                      int64_t M, int64_t h, int64_t V_r, int64_t vocab_start,
                                      float* stats, void* ws, size_t ws_bytes, void* stream) {
    if (!H || !E_r || !targets || !stats) return TP_ERR_NULL;
    if (tp_status s = check_vocab(M, h, V_r)) return s;
    if (!operand_fits(h, true) || ((M + 255) / 256) * ce_ntn(V_r) > kI32 / 8) return TP_ERR_SHAPE;
    if (!ws || ws_bytes < (size_t)ce_tiles_bytes(M, V_r)) return TP_ERR_WORKSPACE;
    if (!aligned16(H) || !aligned16(E_r) || !aligned16(stats) || !aligned16(ws) ||
        (reinterpret_cast<uintptr_t>(targets) & 3))
        return TP_ERR_ALIGN;
    const void* E[1] = {E_r};
    return launched(run_ce_ranks(H, E, 1, targets, M, h, V_r, vocab_start, stats, (float*)ws,
                                 as_stream(stream)));
}

TP_EXPORT tp_status tp_vocab_ce_combine(const float* stats, int P, int64_t M, float* loss,
                                        float* loss_mean, void* stream) {
    if (!stats || !loss) return TP_ERR_NULL;
    if (P <= 0 || M <= 0 || M > kI32) return TP_ERR_SHAPE;
    if (!aligned16(stats) || !aligned16(loss) || (loss_mean && (reinterpret_cast<uintptr_t>(loss_mean) & 3)))
        return TP_ERR_ALIGN;
    return launched(tpk::ce_combine(stats, P, M, loss, loss_mean, as_stream(stream)));
}

TP_EXPORT size_t tp_vocab_parallel_ce_workspace(int64_t M, int64_t V_r, int P) {
    if (M <= 0 || V_r <= 0 || P <= 0) return 0;
    return (size_t)(P * (ce_stats_bytes(M) + ce_tiles_bytes(M, V_r)));
}

TP_EXPORT tp_status tp_vocab_parallel_ce(const void* H, const void* const* E, int P,
                                         const int32_t* targets, int64_t M, int64_t h,
                                         int64_t V_r, float* loss, float* loss_mean, void* ws,
                                         size_t ws_bytes, void* stream) {
    if (!H || !E || !targets || !loss) return TP_ERR_NULL;
    if (P <= 0) return TP_ERR_SHAPE;
    if (tp_status s = check_vocab(M, h, V_r)) return s;
    if (!operand_fits(h, true) || ((M + 255) / 256) * ce_ntn(V_r) > kI32 / 8 ||
        V_r * P > kI32)
        return TP_ERR_SHAPE;
    for (int r = 0; r < P; ++r) {
        if (!E[r]) return TP_ERR_NULL;
        if (!aligned16(E[r])) return TP_ERR_ALIGN;
    }
    if (!ws || ws_bytes < tp_vocab_parallel_ce_workspace(M, V_r, P)) return TP_ERR_WORKSPACE;
    if (!aligned16(H) || !aligned16(loss) || !aligned16(ws) ||
        (reinterpret_cast<uintptr_t>(targets) & 3) ||
        (loss_mean && (reinterpret_cast<uintptr_t>(loss_mean) & 3)))
        return TP_ERR_ALIGN;
    const hipStream_t st = as_stream(stream);
    // ranks' statistics contiguous with stride 3·M floats (the combine's
    // layout), then the tile statistics
    float* stats = (float*)ws;                                   // [P][3][M]
    float* tiles = (float*)((char*)ws + P * ce_stats_bytes(M));  // [P][M][ntn][2]
    if (run_ce_ranks(H, E, P, targets, M, h, V_r, 0, stats, tiles, st)) return TP_ERR_LAUNCH;
    return launched(tpk::ce_combine(stats, P, M, loss, loss_mean, st));
}

TP_EXPORT tp_status tp_layernorm(const void* x, int in, void* y, const void* gamma,
                                 const void* beta, float eps, int64_t M, int64_t h,
                                 void* stream) {
    if (!x || !y) return TP_ERR_NULL;
    if (!is_dtype(in)) return TP_ERR_DTYPE;
    if (M <= 0 || h <= 0 || h % 8 || h > kMaxLnWidthWide || M > kI32 || !(eps > 0.0f))
        return TP_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(y) || (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
        return TP_ERR_ALIGN;
    return launched(tpk::layernorm(x, in == TP_BF16, y, (const float*)gamma, (const float*)beta,
                                   eps, M, h, as_stream(stream)));
}

TP_EXPORT tp_status tp_partial_sum(void* Z, int out, const void* partials, int part, int P,
                                   int64_t M, int64_t h, const void* bias, const void* residual,
                                   int res, void* stream) {
    if (!Z || !partials) return TP_ERR_NULL;
    if (!is_dtype(out) || !is_dtype(part) || (residual && !is_dtype(res))) return TP_ERR_DTYPE;
    if (P <= 0 || M <= 0 || h <= 0 || h % 4 || h > kI32) return TP_ERR_SHAPE;
    if (!aligned16(Z) || !aligned16(partials) || (bias && !aligned16(bias)) ||
        (residual && !aligned16(residual)))
        return TP_ERR_ALIGN;
    if (h <= kMaxLnWidth && M <= kI32)   // one row per workgroup, row in registers
        return launched(tpk::row_sum(Z, out == TP_BF16, partials, part == TP_BF16, P, M, h,
                                     (const float*)bias, residual, residual && res == TP_BF16,
                                     nullptr, nullptr, nullptr, 0.0f, as_stream(stream)));
    return launched(tpk::partial_sum(Z, out == TP_BF16, partials, part == TP_BF16, P, M, h,
                                     (const float*)bias, residual, residual && res == TP_BF16,
                                     as_stream(stream)));
}

TP_EXPORT size_t tp_block_shard_workspace(int64_t b, int64_t s, int64_t h, int64_t H, int64_t d,
                                          int64_t F, int P) {
    if (b <= 0 || s <= 0 || h <= 0 || H <= 0 || d <= 0 || F <= 0 || P <= 0 || H % P || F % P)
        return 0;
    return (size_t)block_ws(b, s, h, H, d, F, P).total;
}

namespace {
// The block; ev_begin / ev_end (both or neither) are recorded on the stream
// around the launches of the MLP's column-parallel GEMM with GeLU.
tp_status block_shard(const void* x, void* out, int out_dtype, void* x1, const void* ln1_g,
                      const void* ln1_b, const void* ln2_g, const void* ln2_b, float eps,
                      const void* const* W_qkv, const void* const* W_o, const void* const* A,
                      const void* const* B, int P, void* ws, size_t ws_bytes, int64_t b,
                      int64_t s, int64_t h, int64_t H, int64_t d, int64_t F, void* stream,
                      hipEvent_t ev_begin, hipEvent_t ev_end) {
    if (!x || !out || !W_qkv || !W_o || !A || !B) return TP_ERR_NULL;
    if (!is_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (P <= 0 || H <= 0 || F <= 0 || H % P || F % P || h != H * d || !(eps > 0.0f))
        return TP_ERR_SHAPE;
    const int64_t M = b * s, Hl = H / P, f = F / P;
    tp_status stat = check_attn_shape(b, s, h, Hl, d);
    if (stat != TP_OK) return stat;
    if (((s + 127) / 128) * (b * H + 7) > kI32) return TP_ERR_SHAPE;
    if (f % 8 || h > kMaxLnWidth || !gemm_bf16_fits(M, f, h, h, f) || !gemm_bf16_fits(M, h, f, f, h))
        return TP_ERR_SHAPE;
    for (int r = 0; r < P; ++r)
        if (!W_qkv[r] || !W_o[r] || !A[r] || !B[r]) return TP_ERR_NULL;
    const void* ptrs[] = {x, out, x1, ln1_g, ln1_b, ln2_g, ln2_b};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return TP_ERR_ALIGN;
    for (int r = 0; r < P; ++r)
        if (!aligned16(W_qkv[r]) || !aligned16(W_o[r]) || !aligned16(A[r]) || !aligned16(B[r]))
            return TP_ERR_ALIGN;
    const BlockWs w = block_ws(b, s, h, H, d, F, P);
    if (!ws || ws_bytes < (size_t)w.total) return TP_ERR_WORKSPACE;
    if (!aligned16(ws)) return TP_ERR_ALIGN;

    const hipStream_t st = as_stream(stream);
    char* base = (char*)ws;
    __bf16* xn = (__bf16*)(base + w.xn);
    float* parts = (float*)(base + w.parts);
    float* x1buf = x1 ? (float*)x1 : (float*)(base + w.x1);
    char* qkv = base + w.qkv;
    char* O = base + w.o;
    char* Y = base + w.y;
    const int64_t n = M * h, HD = Hl * d;
    const int64_t qkv_r = M * 3 * HD, o_r = M * HD, y_r = M * f;     // per-rank elements

    // x1 = x + sum_r Attn_r(LN1(x))
    if (tpk::layernorm(x, true, xn, (const float*)ln1_g, (const float*)ln1_b, eps, M, h, st))
        return TP_ERR_LAUNCH;
    // [Q|K|V]_r = LN1(x)·W_qkv_r for every rank (column-parallel, §3.2)
    if (grouped(P, [&](int) { return (const void*)xn; }, [&](int r) { return W_qkv[r]; },
                [&](int r) { return (void*)(qkv + r * qkv_r * 2); }, h, 3 * HD, 3 * HD,
                M, 3 * HD, h, true, false, st))
        return TP_ERR_LAUNCH;
    // every rank's heads, causal (§3.1), one launch
    if (tpk::attention_fwd(qkv, 3 * HD, O, b, s, Hl, true, st, P, qkv_r, o_r))
        return TP_ERR_LAUNCH;
    // Z_r = O_r·W_o_r, f32 partials (row-parallel, §3.2)
    if (grouped(P, [&](int r) { return (const void*)(O + r * o_r * 2); },
                [&](int r) { return W_o[r]; }, [&](int r) { return (void*)(parts + r * n); },
                HD, h, h, M, h, HD, false, false, st))
        return TP_ERR_LAUNCH;
    // the all-reduce's sum + residual, fused with LN2 of the summed rows
    if (tpk::row_sum(x1buf, false, parts, false, P, M, h, nullptr, x, true, xn,
                     (const float*)ln2_g, (const float*)ln2_b, eps, st))
        return TP_ERR_LAUNCH;
    // out = x1 + sum_r MLP_r(LN2(x1)): Y'_r = GeLU(LN2(x1)·A_r), Z_r = Y'_r·B_r (§2.1)
    if (ev_begin && hipEventRecord(ev_begin, st) != hipSuccess) return TP_ERR_LAUNCH;
    if (grouped(P, [&](int) { return (const void*)xn; }, [&](int r) { return A[r]; },
                [&](int r) { return (void*)(Y + r * y_r * 2); }, h, f, f, M, f, h, true, true, st))
        return TP_ERR_LAUNCH;
    if (ev_end && hipEventRecord(ev_end, st) != hipSuccess) return TP_ERR_LAUNCH;
    if (grouped(P, [&](int r) { return (const void*)(Y + r * y_r * 2); },
                [&](int r) { return B[r]; }, [&](int r) { return (void*)(parts + r * n); },
                f, h, h, M, h, f, false, false, st))
        return TP_ERR_LAUNCH;
    if (tpk::row_sum(out, out_dtype == TP_BF16, parts, false, P, M, h, nullptr, x1buf, false,
                     nullptr, nullptr, nullptr, 0.0f, st))
        return TP_ERR_LAUNCH;
    return TP_OK;
}
}  // namespace

TP_EXPORT tp_status tp_block_shard(const void* x, void* out, int out_dtype, void* x1,
                                   const void* ln1_g, const void* ln1_b, const void* ln2_g,
                                   const void* ln2_b, float eps, const void* const* W_qkv,
                                   const void* const* W_o, const void* const* A,
                                   const void* const* B, int P, void* ws, size_t ws_bytes,
                                   int64_t b, int64_t s, int64_t h, int64_t H, int64_t d,
                                   int64_t F, void* stream) {
    return block_shard(x, out, out_dtype, x1, ln1_g, ln1_b, ln2_g, ln2_b, eps, W_qkv, W_o, A, B,
                       P, ws, ws_bytes, b, s, h, H, d, F, stream, nullptr, nullptr);
}

TP_EXPORT tp_status tp_block_shard_timed(const void* x, void* out, int out_dtype, void* x1,
                                         const void* ln1_g, const void* ln1_b, const void* ln2_g,
                                         const void* ln2_b, float eps, const void* const* W_qkv,
                                         const void* const* W_o, const void* const* A,
                                         const void* const* B, int P, void* ws, size_t ws_bytes,
                                         int64_t b, int64_t s, int64_t h, int64_t H, int64_t d,
                                         int64_t F, void* stream, void* ev_begin, void* ev_end) {
    if (!ev_begin || !ev_end) return TP_ERR_NULL;
    return block_shard(x, out, out_dtype, x1, ln1_g, ln1_b, ln2_g, ln2_b, eps, W_qkv, W_o, A, B,
                       P, ws, ws_bytes, b, s, h, H, d, F, stream, (hipEvent_t)ev_begin,
                       (hipEvent_t)ev_end);
}

TP_EXPORT tp_status tp_probe_mfma(float* out, int blocks, int iters, void* stream) {
    if (!out) return TP_ERR_NULL;
    if (blocks <= 0 || iters <= 0) return TP_ERR_SHAPE;
    if (!aligned16(out)) return TP_ERR_ALIGN;
    return launched(tpk::mfma_probe(out, blocks, iters, as_stream(stream)));
}
