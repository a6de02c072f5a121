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
 * Conventions: every array is row-major float64.  Every sum runs in
 * ascending index order.  No blocking, fusion or reordering: each function is
 * the definition written out.  The matrix products of the path (X·W) are not
 * here: the Python side takes them from a library float64 matmul and composes
 * them with these functions.
 *
 * OpenMP is used only to spread independent rows over host cores; it does
 * not change any per-element arithmetic or its order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

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

/* Derivative of the exact GeLU, by the product rule on x·Phi(x):
 *   d/dx GeLU(x) = Phi(x) + x·phi(x),  phi(x) = exp(-x^2/2)/sqrt(2 pi),
 * the standard normal density (Phi' = phi).  Needed by the backward pass of
 * the MLP share: the gradient of Y'_i = GeLU(Y_i) is taken locally on each
 * rank, exactly as the forward GeLU is ([Megatron explainer] §2.2). */
EXPORT double orc_gelu_grad(double x)
{
    const double Phi = 0.5 * (1.0 + erf(x / sqrt(2.0)));
    const double phi = exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0));
    return Phi + x * phi;
}

EXPORT void orc_gelu_grad_inplace(double* y, int64_t n)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_gelu_grad(y[i]);
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

/* Scaled dot-product attention of the local heads for chosen query rows of
 * one sequence, [Megatron explainer] §3.1; per-head formula as in the
 * [Operator-split article] (scores / sqrt(d_k), masked to -inf, softmax, ·V).
 *
 * Q     [nq, Hl·d]   the queries' projections (local head j: columns j·d..)
 * K, V  [L, Hl·d]    the sequence's key/value projections, tokens 0..L-1
 * tpos  [nq]         position of each query in the sequence (< L)
 * O     [nq, Hl·d]   heads concatenated along the feature axis
 *
 * For head j and query at position t:
 *   sigma_u = (q · k_u) / sqrt(d)   for u in 0..L-1 (only u <= t if causal)
 *   mu = max_u sigma_u,  p_u = exp(sigma_u - mu),
 *   o = (sum_u p_u · v_u) / (sum_u p_u)
 * -- the textbook two-pass stable softmax; every sum is in ascending u. */
EXPORT void orc_attention_rows(const double* Q, const double* K, const double* V,
                               const int64_t* tpos, int64_t nq, int64_t L,
                               int64_t Hl, int64_t d, int causal, double* O)
{
    const int64_t HD = Hl * d;
    const double scale = 1.0 / sqrt((double)d);
    #pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < nq; ++i) {
        const int64_t nk = causal ? tpos[i] + 1 : L;
        double* sc = (double*)malloc(sizeof(double) * (size_t)nk);
        for (int64_t j = 0; j < Hl; ++j) {
            const double* q = Q + i * HD + j * d;
            double mx = -INFINITY;
            for (int64_t u = 0; u < nk; ++u) {
                double acc = 0.0;
                for (int64_t c = 0; c < d; ++c) acc += q[c] * K[u * HD + j * d + c];
                sc[u] = acc * scale;
                if (sc[u] > mx) mx = sc[u];
            }
            double den = 0.0;
            for (int64_t u = 0; u < nk; ++u) { sc[u] = exp(sc[u] - mx); den += sc[u]; }
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t u = 0; u < nk; ++u) acc += sc[u] * V[u * HD + j * d + c];
                O[i * HD + j * d + c] = acc / den;
            }
        }
        free(sc);
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
