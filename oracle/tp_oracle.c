/*
 * tp_oracle.c -- plain, slow, fp64 CPU oracle for one tensor-parallel rank's
 * share of a Megatron-style Transformer block.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Sources (cited by short name below):
 *   [Megatron explainer] "图解Transformer并行计算：从矩阵乘法切分到Megatron架构设计",
 *       un.csdn.net/7y5fj9k05scw -- the authority for what is computed.
 *   [PyTorch TP tutorial] the PyTorch tensor-parallel tutorial page at
 *       hotelren.com/news/6074135 (section 3.3 assembles the pre-LN block).
 *   [Operator-split article] "5.1 Tensor并行与算子拆分", aiknowledge.cn
 *       (class TensorParallelMultiheadAttention: the per-head attention formula).
 *
 * Conventions: every array is row-major float64; a weight W of a linear layer
 * has shape [in, out] and the layer computes X·W (the [Megatron explainer] §1
 * convention Y = X @ W with W of shape [h, h']).  Every sum over a
 * contraction index runs in ascending index order.  No blocking, fusion or
 * reordering: each function is the definition written out.
 *
 * OpenMP is used only to spread independent output rows over host cores; it
 * does not change any per-element arithmetic or its order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* Y[M,N] = X[M,K] · W[K,N]  (+ bias[N] when bias != NULL).
 * [Megatron explainer] §1: Y = X @ W.  Leading dimensions allow the caller to
 * pass column slices (W_i = W[:, r·c:(r+1)·c]) without copying.
 * Each Y[m,n] = sum_{k=0}^{K-1} X[m,k]·W[k,n], k ascending, then + bias[n]. */
EXPORT void orc_matmul(const double* X, int64_t ldx, const double* W, int64_t ldw,
                       const double* bias, double* Y, int64_t ldy,
                       int64_t M, int64_t K, int64_t N)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double* y = Y + m * ldy;
        for (int64_t n = 0; n < N; ++n) y[n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xk = X[m * ldx + k];
            const double* w = W + k * ldw;
            for (int64_t n = 0; n < N; ++n) y[n] += xk * w[n];
        }
        if (bias)
            for (int64_t n = 0; n < N; ++n) y[n] += bias[n];
    }
}

/* GeLU in its exact form x·Phi(x) = x/2·(1 + erf(x/sqrt 2)), where Phi is the
 * standard normal CDF.  [Megatron explainer] §2 names GeLU as the MLP's
 * activation; the tutorial's block uses nn.GELU() whose default is this exact
 * (non-tanh) form. */
EXPORT double orc_gelu(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

EXPORT void orc_gelu_inplace(double* y, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_gelu(y[i]);
}

/* One rank's MLP share, [Megatron explainer] §2.1 / §2.2:
 *   Y_i = X·A_i (+ a_i),   Y'_i = GeLU(Y_i)  (local, no communication),
 *   Z_i = Y'_i·B_i          (a partial sum; the full Z is sum_i Z_i).
 * X [M,h], A_i [h,f], a_i [f] or NULL, B_i [f,h], Z_i [M,h]. */
EXPORT void orc_mlp_shard(const double* X, const double* A_i, const double* a_i,
                          const double* B_i, double* Z_i,
                          int64_t M, int64_t h, int64_t f)
{
    double* Y = (double*)malloc(sizeof(double) * (size_t)(M * f));
    orc_matmul(X, h, A_i, f, a_i, Y, f, M, h, f);
    orc_gelu_inplace(Y, M * f);
    orc_matmul(Y, f, B_i, h, NULL, Z_i, h, M, f, h);
    free(Y);
}

/* LayerNorm over the last dimension (the tutorial block's nn.LayerNorm(h)):
 *   mu = (1/h) sum_c x_c,  var = (1/h) sum_c (x_c - mu)^2  (population form),
 *   y_c = (x_c - mu) / sqrt(var + eps) · gamma_c + beta_c.
 * gamma/beta may be NULL (meaning 1 and 0). */
EXPORT void orc_layernorm(const double* x, const double* gamma, const double* beta,
                          double eps, double* y, int64_t M, int64_t h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const double* xr = x + m * h;
        double* yr = y + m * h;
        double mu = 0.0;
        for (int64_t c = 0; c < h; ++c) mu += xr[c];
        mu /= (double)h;
        double var = 0.0;
        for (int64_t c = 0; c < h; ++c) var += (xr[c] - mu) * (xr[c] - mu);
        var /= (double)h;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < h; ++c) {
            double v = (xr[c] - mu) * inv;
            if (gamma) v *= gamma[c];
            if (beta) v += beta[c];
            yr[c] = v;
        }
    }
}

/* One rank's attention share for a chosen set of output rows,
 * [Megatron explainer] §3.1 and §3.2; per-head formula as in the
 * [Operator-split article] (scores / sqrt(d_k), masked to -inf, softmax, ·V).
 *
 * X        [b·s, h], token m = beta·s + t.
 * Wqkv     [h, 3·Hl·d]: columns [0,Hl·d) are this rank's W_q slice, then W_k,
 *          then W_v; local head j owns columns j·d..j·d+d-1 of each block.
 * Wo       [Hl·d, h]: this rank's row slice of W_o.
 * rows     nrows token indices whose output rows are wanted (any order).
 * Z        [nrows, h]: Z[i] = O[rows[i]] · Wo, where O concatenates the local
 *          heads' outputs along the feature axis.
 *
 * For head j and query token t of sequence beta:
 *   sigma_u = (q_t · k_u) / sqrt(d)    for keys u in 0..s-1 (u <= t if causal)
 *   mu = max_u sigma_u,  p_u = exp(sigma_u - mu),
 *   o_t = (sum_u p_u · v_u) / (sum_u p_u).
 * The keys and values needed are those of the query's own sequence: the oracle
 * projects exactly the prefix it uses (all s tokens when not causal). */
EXPORT void orc_attn_shard_rows(const double* X, int64_t b, int64_t s, int64_t h,
                                const double* Wqkv, const double* Wo,
                                int64_t Hl, int64_t d, int causal,
                                const int64_t* rows, int64_t nrows, double* Z)
{
    const int64_t W3 = 3 * Hl * d, HD = Hl * d;
    const double scale = 1.0 / sqrt((double)d);
    for (int64_t beta = 0; beta < b; ++beta) {
        /* longest prefix any requested row of this sequence needs */
        int64_t L = 0;
        for (int64_t i = 0; i < nrows; ++i) {
            if (rows[i] / s != beta) continue;
            int64_t need = causal ? (rows[i] % s) + 1 : s;
            if (need > L) L = need;
        }
        if (L == 0) continue;
        /* K and V of tokens 0..L-1: K = X·W_k, V = X·W_v */
        double* KV = (double*)malloc(sizeof(double) * (size_t)(L * 2 * HD));
        orc_matmul(X + beta * s * h, h, Wqkv + HD, W3, NULL, KV, 2 * HD, L, h, 2 * HD);
        #pragma omp parallel for schedule(dynamic)
        for (int64_t i = 0; i < nrows; ++i) {
            if (rows[i] / s != beta) continue;
            const int64_t t = rows[i] % s;
            const int64_t nk = causal ? t + 1 : s;
            double* q = (double*)malloc(sizeof(double) * (size_t)HD);
            double* o = (double*)malloc(sizeof(double) * (size_t)HD);
            double* sc = (double*)malloc(sizeof(double) * (size_t)nk);
            /* q = X[token] · W_q */
            for (int64_t n = 0; n < HD; ++n) q[n] = 0.0;
            for (int64_t k = 0; k < h; ++k) {
                const double xk = X[(beta * s + t) * h + k];
                for (int64_t n = 0; n < HD; ++n) q[n] += xk * Wqkv[k * W3 + n];
            }
            for (int64_t j = 0; j < Hl; ++j) {
                double mx = -INFINITY;
                for (int64_t u = 0; u < nk; ++u) {
                    double acc = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        acc += q[j * d + c] * KV[u * 2 * HD + j * d + c];
                    sc[u] = acc * scale;
                    if (sc[u] > mx) mx = sc[u];
                }
                double den = 0.0;
                for (int64_t u = 0; u < nk; ++u) { sc[u] = exp(sc[u] - mx); den += sc[u]; }
                for (int64_t c = 0; c < d; ++c) {
                    double acc = 0.0;
                    for (int64_t u = 0; u < nk; ++u)
                        acc += sc[u] * KV[u * 2 * HD + HD + j * d + c];
                    o[j * d + c] = acc / den;
                }
            }
            /* Z row = O · W_o  (row-parallel partial product, §3.2) */
            double* z = Z + i * h;
            for (int64_t n = 0; n < h; ++n) z[n] = 0.0;
            for (int64_t k = 0; k < HD; ++k) {
                const double ok = o[k];
                for (int64_t n = 0; n < h; ++n) z[n] += ok * Wo[k * h + n];
            }
            free(q); free(o); free(sc);
        }
        free(KV);
    }
}

/* The one-GPU stand-in for the all-reduce, [Megatron explainer] §1.1 and §2.1
 * (Z = Z1 + Z2): Z = sum_{r=0}^{P-1} parts[r] (r ascending), then + bias[col]
 * (the row-parallel bias, added once after the sum) and + residual, each only
 * when non-NULL.  parts is [P][M·h] contiguous, bias [h], residual [M·h]. */
EXPORT void orc_partial_sum(const double* parts, int64_t P, int64_t M, int64_t h,
                            const double* bias, const double* residual, double* Z)
{
    const int64_t n = M * h;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int64_t r = 0; r < P; ++r) acc += parts[r * n + i];
        if (bias) acc += bias[i % h];
        if (residual) acc += residual[i];
        Z[i] = acc;
    }
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of host threads the loops above spread over. */
EXPORT int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
