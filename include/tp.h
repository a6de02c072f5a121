/*
 * tp.h -- C ABI of libtp.so: one tensor-parallel rank's share of a
 * Megatron-style Transformer block, computed on one MI355X (gfx950).
 *
 * Sources cited below by short name:
 *   [Megatron explainer] "图解Transformer并行计算：从矩阵乘法切分到Megatron架构设计"
 *       (un.csdn.net/7y5fj9k05scw): §1.1 row split, §1.2 column split,
 *       §2.1/§2.2 the MLP, §3.1/§3.2 head-sharded attention.
 *   [PyTorch TP tutorial] hotelren.com/news/6074135, section 3.3 (the
 *       pre-LN block: x + attention(norm1(x)), then x + mlp(norm2(x))),
 *       section 2.2 (heads per rank = num_heads / world_size) and section 3.2
 *       (a shape that does not divide by the world size is rejected).
 *   [ops-transformer] intelliparadigm.com/article/weixin_42537919/2252113,
 *       §3.1 (attention parallelisation: strategy B, K/V split along the
 *       feature dimension, partial scores combined across devices).
 *
 * Conventions shared by every entry point:
 *  - Matrices are row-major with the X·W convention: a weight of a linear
 *    layer has shape [in, out].  "M" is the token count b·s; token m is
 *    position t = m % s of sequence m / s.
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc / PyTorch memory)
 *    owned by the caller, 16-byte aligned.  Host pointers are only the arrays
 *    of per-rank device pointers taken by tp_block_shard and
 *    tp_linear_batched.
 *  - The library never allocates, frees or synchronises.  All work is
 *    enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream); outputs are ready when that stream reaches this point.
 *  - Arguments are validated before anything is launched; on any error the
 *    call returns a non-zero tp_status and touches no memory.  TP_ERR_LAUNCH
 *    reports a failed kernel launch (hipGetLastError after enqueueing), in
 *    which case outputs are unspecified.
 *  - Calls are reentrant; calls that share a workspace on different streams
 *    race.
 */
#ifndef TP_H
#define TP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_status {
    TP_OK = 0,
    TP_ERR_NULL = 1,      /* a required pointer is NULL                          */
    TP_ERR_SHAPE = 2,     /* a size is <= 0, does not divide, or is unsupported  */
    TP_ERR_DTYPE = 3,     /* dtype code not accepted by this entry point         */
    TP_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                    */
    TP_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the *_workspace size */
    TP_ERR_LAUNCH = 6,    /* the HIP runtime rejected a kernel launch            */
    TP_ERR_SCRATCH = 7    /* too large for the fixed scratch of an allocation-free
                             entry point (tp_mlp_shard_noalloc)                  */
} tp_status;

typedef enum tp_dtype {
    TP_F32 = 0,   /* IEEE binary32                                   */
    TP_BF16 = 1   /* bfloat16 (top 16 bits of binary32), RNE rounded */
} tp_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* tp_status_string(int status);

/* ABI version of this header: 2 (tp_matmul_grouped took its optional
 * workspace arguments in version 2). */
int tp_abi_version(void);

/* ------------------------------------------------------------------------
 * tp_mlp_shard -- one rank's MLP share.  [Megatron explainer] §2.1, §2.2:
 * the first linear layer is split by columns, GeLU is applied locally, the
 * second is split by rows, and the result is a partial sum that the
 * all-reduce would add over ranks:
 *     Y_i = X·A_i + a_i,    Y'_i = GeLU(Y_i) = Y_i/2·(1+erf(Y_i/sqrt 2)),
 *     Z_i = Y'_i·B_i.
 *   X   [M,h]  in dtype `in`          A_i [h,f] in dtype `in`
 *   a_i [f]    f32, or NULL for none  B_i [f,h] in dtype `in`
 *   Z_i [M,h]  in dtype `out` (accumulated in f32)
 *   ws  >= tp_mlp_shard_workspace(M, f, in) bytes (holds Y'_i in dtype `in`).
 * in: TP_BF16 (MFMA path, f32 accumulate, Y'_i rounded to bf16) or TP_F32
 * (f32 FMA path).  out: TP_F32 or TP_BF16.  bf16 needs h % 8 == 0 and
 * f % 8 == 0.
 * ---------------------------------------------------------------------- */
size_t tp_mlp_shard_workspace(int64_t M, int64_t f, int in);
tp_status tp_mlp_shard(const void* X, const void* A_i, const void* a_i, const void* B_i,
                       void* Z_i, void* ws, size_t ws_bytes,
                       int64_t M, int64_t h, int64_t f, int in, int out, void* stream);

/* tp_mlp_shard_noalloc -- tp_mlp_shard for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and precision as
 * tp_mlp_shard (bit for bit), with no workspace argument: Y'_i lives in a
 * fixed 64 MiB device array inside the library, which every GPU the library
 * runs on holds until the process ends.  The share runs on blocks of token
 * rows whose Y'_i fits that array (rows are independent), so any M is
 * accepted; f is limited to f·256·sizeof(in) <= 64 MiB (f <= 131072 for
 * TP_BF16, 65536 for TP_F32), else TP_ERR_SCRATCH before anything is
 * launched.  The call allocates and frees nothing and never synchronises.
 * All calls on one GPU share its array and nothing in it needs to start at
 * zero; calls that overlap on one GPU (two streams, two host threads) race
 * on it and must be ordered by the caller. */
tp_status tp_mlp_shard_noalloc(const void* X, const void* A_i, const void* a_i,
                               const void* B_i, void* Z_i, int64_t M, int64_t h, int64_t f,
                               int in, int out, void* stream);

/* ------------------------------------------------------------------------
 * Training: the MLP share's forward keeping its activations, and its
 * backward.  [Megatron explainer] §2.2: the backward mirrors the forward;
 * every rank receives the same dZ = ∂L/∂Z, computes the gradients of its own
 * A_i, B_i by the chain rule through Z_i = GeLU(X·A_i + a_i)·B_i, and forms a
 * local input gradient dX_i whose sum over ranks, one all-reduce, is ∂L/∂X
 * (tp_partial_sum stands in for that all-reduce):
 *     dY'_i = dZ·B_i^T,   dY_i = dY'_i ⊙ GeLU'(Y_i),
 *     dB_i = Y'_i^T·dZ,   dA_i = X^T·dY_i,   da_i = Σ_rows dY_i,
 *     dX_i = dY_i·A_i^T   (dX = Σ_i dX_i).
 * bf16 operands only (the MFMA path), h % 8 == 0 and f % 8 == 0.
 *
 * tp_mlp_shard_train_fwd -- Z_i as tp_mlp_shard, also storing
 *   Y_i  [M,f] bf16: the pre-activation X·A_i + a_i,
 *   Yp_i [M,f] bf16: GeLU(Y_i) (the second GEMM's input),
 * which tp_mlp_shard_backward takes back.  Z_i in dtype `out`. */
tp_status tp_mlp_shard_train_fwd(const void* X, const void* A_i, const void* a_i,
                                 const void* B_i, void* Z_i, void* Y_i, void* Yp_i,
                                 int64_t M, int64_t h, int64_t f, int out, void* stream);

/* tp_mlp_shard_backward -- the gradients above from the saved Y_i, Yp_i.
 *   X [M,h], A_i [h,f], B_i [f,h], Y_i, Yp_i [M,f], dZ [M,h]: bf16 inputs
 *   dX_i [M,h] in dtype `dx_dtype` (TP_F32 or TP_BF16): this rank's partial
 *   dA_i [h,f], dB_i [f,h]: f32;  da_i [f] f32, or NULL to skip it
 *   ws >= tp_mlp_shard_backward_workspace(M, f) bytes (dY_i in bf16 and the
 *        bias gradient's per-chunk partial sums).
 * The bias gradient is summed in a fixed order: results are bitwise
 * reproducible from run to run. */
size_t tp_mlp_shard_backward_workspace(int64_t M, int64_t f);
tp_status tp_mlp_shard_backward(const void* X, const void* A_i, const void* B_i,
                                const void* Y_i, const void* Yp_i, const void* dZ,
                                void* dX_i, void* dA_i, void* dB_i, void* da_i, void* ws,
                                size_t ws_bytes, int64_t M, int64_t h, int64_t f,
                                int dx_dtype, void* stream);

/* ------------------------------------------------------------------------
 * tp_attn_shard -- one rank's attention share.  [Megatron explainer] §3.1,
 * §3.2: the Q, K and V projections are split by columns so that this rank
 * owns H_l whole heads, each head computes softmax(Q·K^T/sqrt d)·V locally,
 * and W_o is split by rows so the rank's output is a partial sum:
 *     [Q|K|V] = X·W_qkv_i,   O_j = softmax(Q_j·K_j^T/sqrt(d) + mask)·V_j,
 *     Z_i = [O_0|...|O_{H_l-1}]·W_o_i.
 *   X       [b·s, h] bf16
 *   W_qkv_i [h, 3·H_l·d] bf16, columns [W_q | W_k | W_v] of this rank's heads;
 *           inside each block local head j owns columns j·d .. j·d+d-1
 *   W_o_i   [H_l·d, h] bf16 (this rank's row block of W_o)
 *   Z_i     [b·s, h] in dtype `out` (TP_F32 or TP_BF16)
 *   causal  non-zero: key u is visible to query t iff u <= t
 *   ws      >= tp_attn_shard_workspace(b, s, H_l, d) bytes
 * d must be 128 (the kernel's head tile); h % 8 == 0.
 * ---------------------------------------------------------------------- */
size_t tp_attn_shard_workspace(int64_t b, int64_t s, int64_t H_l, int64_t d);
tp_status tp_attn_shard(const void* X, const void* W_qkv_i, const void* W_o_i, void* Z_i,
                        void* ws, size_t ws_bytes, int64_t b, int64_t s, int64_t h,
                        int64_t H_l, int64_t d, int causal, int out, void* stream);

/* ------------------------------------------------------------------------
 * Training: the attention share's forward keeping its activations, and its
 * backward.  [Megatron explainer] §3.2 (backward): dZ = ∂L/∂Z reaches every
 * rank; each computes the gradients of its own W_o,i and W_qkv,i and a local
 * input gradient whose sum over ranks (one all-reduce) is ∂L/∂X:
 *     dO = dZ·W_o,i^T,   dW_o,i = O_i^T·dZ,
 *     (dQ, dK, dV) = tp_attention_core_backward(...),
 *     dW_qkv,i = X^T·[dQ|dK|dV],   dX_i = [dQ|dK|dV]·W_qkv,i^T.
 *
 * tp_attn_shard_train_fwd -- Z_i as tp_attn_shard, also storing
 *   qkv [b·s, 3·H_l·d] bf16, O [b·s, H_l·d] bf16 and lse f32 [b·H_l·s]
 * (see tp_attention_core_train), which the backward takes back. */
tp_status tp_attn_shard_train_fwd(const void* X, const void* W_qkv_i, const void* W_o_i,
                                  void* Z_i, void* qkv, void* O, float* lse, int64_t b, int64_t s,
                                  int64_t h, int64_t H_l, int64_t d, int causal, int out,
                                  void* stream);

/* tp_attn_shard_backward -- the gradients above.
 *   X [b·s, h], W_qkv_i [h, 3·H_l·d], W_o_i [H_l·d, h], dZ [b·s, h]: bf16
 *   qkv, O, lse: from tp_attn_shard_train_fwd
 *   dX_i [b·s, h] in dtype `dx_dtype` (this rank's partial);
 *   dW_qkv_i [h, 3·H_l·d], dW_o_i [H_l·d, h]: f32
 *   ws >= tp_attn_shard_backward_workspace(b, s, H_l, d) bytes (dO, dqkv, D).
 * The two weight gradients run as one grouped launch (tp_matmul_grouped's),
 * given the dO part of ws once dO is consumed: where its last wave of tiles
 * fills at most half the GPU, those tiles' sums over the b·s tokens are split
 * into two (or four) ordered partial sums.  Results are deterministic for a
 * given device and shape. */
size_t tp_attn_shard_backward_workspace(int64_t b, int64_t s, int64_t H_l, int64_t d);
tp_status tp_attn_shard_backward(const void* X, const void* W_qkv_i, const void* W_o_i,
                                 const void* qkv, const void* O, const float* lse,
                                 const void* dZ, void* dX_i, void* dW_qkv_i, void* dW_o_i,
                                 void* ws, size_t ws_bytes, int64_t b, int64_t s, int64_t h,
                                 int64_t H_l, int64_t d, int causal, int dx_dtype, void* stream);

/* ------------------------------------------------------------------------
 * tp_partial_sum -- the arithmetic of the all-reduce on one GPU.
 * [Megatron explainer] §1.1 (row split: the partial products are summed) and
 * §2.1 (Z = Z1 + Z2):
 *     Z = sum_{r=0}^{P-1} partials[r]  (+ bias[col])  (+ residual),
 * summed in f32 in ascending r, so results are bit-reproducible.
 *   partials  [P][M·h] contiguous, dtype `part` (TP_F32 or TP_BF16)
 *   bias      [h] f32 or NULL (a row-parallel bias, added once)
 *   residual  [M,h] dtype `res` or NULL
 *   Z         [M,h] dtype `out`; may alias `residual` when both are f32.
 * Needs h % 4 == 0.
 * ---------------------------------------------------------------------- */
tp_status tp_partial_sum(void* Z, int out, const void* partials, int part, int P,
                         int64_t M, int64_t h, const void* bias,
                         const void* residual, int res, void* stream);

/* ------------------------------------------------------------------------
 * tp_block_shard -- a whole pre-LN Transformer block with all P ranks'
 * shares emulated on this GPU ([PyTorch TP tutorial] 3.3):
 *     x1  = x  + sum_r Attn_r(LN1(x))       (the attention all-reduce)
 *     out = x1 + sum_r MLP_r(LN2(x1))       (the MLP all-reduce)
 * with Attn_r and MLP_r the tp_attn_shard / tp_mlp_shard shares of rank r
 * (H_l = H/P heads, f = F/P columns of A), causal attention, no biases.
 * Each step runs as one launch over all ranks (the ranks' products have one
 * shape; each rank still uses only its own slices and writes its own f32
 * partial), and the sum over ranks is taken in ascending rank order, f32,
 * then the residual; LN2 is fused into the first sum.
 *   x      [b·s, h] bf16           out  [b·s, h] dtype `out`
 *   x1     [b·s, h] f32 or NULL    (if given, receives the residual stream
 *                                   after attention)
 *   ln*_g, ln*_b  [h] f32 or NULL (gamma=1, beta=0); eps > 0
 *   W_qkv, W_o, A, B  HOST arrays of P device pointers: rank r's
 *                     [h,3·H_l·d], [H_l·d,h], [h,f], [f,h] bf16 slices
 *   ws     >= tp_block_shard_workspace(b, s, h, H, d, F, P) bytes
 * Needs h == H·d, H % P == 0, F % P == 0, d == 128, h % 8 == 0, f % 8 == 0.
 * ---------------------------------------------------------------------- */
size_t tp_block_shard_workspace(int64_t b, int64_t s, int64_t h, int64_t H, int64_t d,
                                int64_t F, int P);
tp_status tp_block_shard(const void* x, void* out, int out_dtype, void* x1,
                         const void* ln1_g, const void* ln1_b,
                         const void* ln2_g, const void* ln2_b, float eps,
                         const void* const* W_qkv, const void* const* W_o,
                         const void* const* A, const void* const* B, int P,
                         void* ws, size_t ws_bytes, int64_t b, int64_t s, int64_t h,
                         int64_t H, int64_t d, int64_t F, void* stream);

/* ========================================================================
 * Component entry points: the individual steps of the path, exported so
 * that each can be checked on its own.
 * ====================================================================== */

/* Epilogues of tp_linear (NONE, GELU) and tp_matmul (all four). */
typedef enum tp_epilogue {
    TP_EPI_NONE = 0,     /* C = X·W (+bias)                                    */
    TP_EPI_GELU = 1,     /* C = GeLU(X·W + bias), exact erf form (§2.1's GeLU) */
    TP_EPI_GELU_BWD = 2, /* C = (X·W + bias) ⊙ GeLU'(aux): the chain rule
                            through the GeLU, aux = the saved pre-activation   */
    TP_EPI_GELU_SAVE = 3 /* C = GeLU(X·W + bias) and aux = X·W + bias, both bf16:
                            the training forward keeps what the backward needs */
} tp_epilogue;

/* tp_linear -- C[M,N] = epi(X[M,K]·W[K,N] + bias[N]) with an f32 accumulator.
 * [Megatron explainer] §1: Y = X·W, the product every split applies to its
 * block.  Row-major with leading dimensions ldx, ldw, ldc (in elements).
 *   in : TP_BF16 (MFMA) or TP_F32;  out: TP_F32 or TP_BF16;  bias f32 or NULL.
 * bf16 needs K % 8 == 0, N % 8 == 0 and leading dimensions that are
 * multiples of 8. */
tp_status tp_linear(const void* X, int64_t ldx, const void* W, int64_t ldw,
                    const void* bias, void* C, int64_t ldc,
                    int64_t M, int64_t N, int64_t K, int in, int out, int epilogue,
                    void* stream);

/* tp_linear_batched -- `count` independent products of one shape in one
 * launch: C[g] = epi(X[g]·W[g] + bias[g]) for g = 0 .. count-1, each as in
 * tp_linear.  X, W, C (and bias, which may be NULL as a whole or per entry)
 * are HOST arrays of `count` device pointers; a pointer may repeat (e.g. the
 * same X for every rank's column-parallel product).  This is how one GPU runs
 * the identical per-rank products of several emulated tensor-parallel ranks
 * ([Megatron explainer] §2.1, §3.2: every rank applies the same operation to
 * its own slice) without a tail per rank.  bf16 inputs run as one grouped
 * MFMA launch per 32 products; f32 inputs run one product after another. */
tp_status tp_linear_batched(const void* const* X, int64_t ldx, const void* const* W,
                            int64_t ldw, const void* const* bias, void* const* C, int64_t ldc,
                            int count, int64_t M, int64_t N, int64_t K, int in, int out,
                            int epilogue, void* stream);

/* tp_matmul -- C[M,N] = epi(op(A)·op(B) + bias[N]) on bf16 operands with an
 * f32 accumulator, where op(A) = A [M,K] (trans_a = 0) or A^T for A stored
 * [K,M] (trans_a = 1), and op(B) = B [K,N] (trans_b = 0) or B^T for B stored
 * [N,K] (trans_b = 1).  The backward of the column- and row-parallel layers
 * ([Megatron explainer] §2.2) needs both transposed forms: the input gradient
 * dY·W^T (trans_b) and the weight gradient X^T·dY (trans_a).  No operand is
 * transposed in memory.  Row-major storage, leading dimensions in elements.
 * Supported (trans_a, trans_b, epilogue):
 *     (0,0) NONE, GELU (out f32 or bf16), GELU_SAVE (out bf16);
 *     (0,1) NONE, GELU_BWD (out f32 or bf16);
 *     (1,0) NONE (out f32 or bf16);
 * anything else is TP_ERR_DTYPE.
 *   aux  [M,N] bf16 with leading dimension ldaux: read by GELU_BWD, written by
 *        GELU_SAVE, ignored (may be NULL) otherwise.
 *   bias f32 [N] or NULL.
 * The contiguous dimension of every operand and of C must be a multiple of 8
 * (K for a K-contiguous operand, M or N otherwise) and so must every leading
 * dimension. */
tp_status tp_matmul(const void* A, int64_t lda, int trans_a, const void* B, int64_t ldb,
                    int trans_b, const void* bias, void* C, int64_t ldc, void* aux,
                    int64_t ldaux, int64_t M, int64_t N, int64_t K, int out, int epilogue,
                    void* stream);

/* tp_matmul_grouped -- `count` (1..16) products C[g] = op(A[g])·op(B[g]) of
 * one layout (trans_a, trans_b as in tp_matmul, no epilogue), one output
 * dtype and one inner size K, each with its own M[g], N[g] and leading
 * dimensions, in a single launch.  A backward pass's weight gradients
 * ([Megatron explainer] §2.2, §3.2: every rank forms the gradients of its
 * own weight slices) are such a set: launched together, one product's tiles
 * fill the partly idle last wave of the other's.  A, lda, B, ldb, C, ldc,
 * M, N are HOST arrays of `count` entries (device pointers, sizes); each
 * group must satisfy tp_matmul's conditions.
 *   ws, ws_bytes: optional device memory (16-byte aligned; NULL for none)
 *     that the launch may use, f32 output only: when its last wave of
 *     workgroups fills at most half (a quarter) of the compute units and
 *     K >= 4096 (8192), each tile of that wave runs as 2 (4) workgroups over
 *     equal K ranges, the first writing C, the others a block of ws each,
 *     and a second launch adds those blocks to C in range order.  Results
 *     stay deterministic for a given device, shapes and ws_bytes; they can
 *     differ in the last bits from a launch without ws (the sum over K is
 *     split in two (four) partial sums).  ws is not read before it is
 *     written and may hold anything. */
tp_status tp_matmul_grouped(const void* const* A, const int64_t* lda, int trans_a,
                            const void* const* B, const int64_t* ldb, int trans_b,
                            void* const* C, const int64_t* ldc, const int64_t* M,
                            const int64_t* N, int count, int64_t K, int out, void* ws,
                            size_t ws_bytes, void* stream);

/* tp_gemm_tile_cols -- the output-tile width, in columns, that the bf16 GEMM
 * behind tp_linear, tp_linear_batched, tp_matmul and tp_matmul_grouped uses
 * for a launch of `count` products (host arrays M[count], N[count]) with
 * inner size K, layout (trans_a, trans_b) and epilogue as in tp_matmul, on
 * the current device: 128 when no product is wider than 128 columns, else
 * 256, or 192 or 384 where fewer or better-filled waves of workgroups make
 * the launch faster.  The width changes the speed only,
 * never a result: every output element sees the same MFMA sequence over K.
 * Host logic only (nothing is launched); with no GPU present it answers for
 * 256 compute units.  Returns 0 for invalid arguments (count outside 1..16,
 * a size <= 0, both operands transposed, an unknown epilogue). */
int tp_gemm_tile_cols(int trans_a, int trans_b, int epilogue, int count, const int64_t* M,
                      const int64_t* N, int64_t K);

/* tp_attention_kv_split -- attention with Q, K and V split along the feature
 * dimension over P emulated ranks ("strategy B", K/V splitting, of the
 * ops-transformer article [ops-transformer] §3.1): rank r holds the features
 * F_r = [r·d/P, (r+1)·d/P) of every head's Q, K and V, computes the partial
 * scores S_r = Q_r·K_r^T (the exchange step sums them over the ranks before
 * the softmax, which is not linear), and forms its feature slice of the head
 * output, O[:, F_r] = softmax(S/sqrt(d) + causal mask)·V_r.  The partial
 * scores are materialised in f32 ([s, s] per rank and head, stored as
 * 128x128 tiles, s rounded up to a multiple of 128), the softmax
 * weights in bf16 (unnormalised, the row maximum's weight exactly 1), the
 * products with V in f32, divided by the sum of the same rounded weights;
 * (sequence, head) pairs run 32 at a time.
 *   qkv  [b·s, ld_qkv] bf16, columns [Q | K | V], each H·d wide, head-major
 *   O    [b·s, ldo] bf16: head h's features at columns h·d .. h·d + d - 1, the
 *        ranks' slices in rank order
 *   ws   >= tp_attention_kv_split_workspace(b, s, H, d, P) bytes
 * Needs d % P == 0, (d/P) % 8 == 0, s % 8 == 0, s <= 8192, ld_qkv >= 3·H·d and
 * ldo >= H·d (both multiples of 8); otherwise TP_ERR_SHAPE. */
size_t    tp_attention_kv_split_workspace(int64_t b, int64_t s, int64_t H, int64_t d, int P);
tp_status tp_attention_kv_split(const void* qkv, int64_t ld_qkv, void* O, int64_t ldo,
                                int64_t b, int64_t s, int64_t H, int64_t d, int P, int causal,
                                void* ws, size_t ws_bytes, void* stream);

/* tp_attention_core -- per (sequence, local head) softmax(Q·K^T/sqrt d)·V
 * ([Megatron explainer] §3.1) on projections already in memory.
 *   qkv [b·s, ld_qkv] bf16: for local head j, Q at columns j·d, K at
 *       H_l·d + j·d, V at 2·H_l·d + j·d (d contiguous columns each)
 *   O   [b·s, H_l·d] bf16, heads concatenated along the feature axis.
 * d must be 128; ld_qkv >= 3·H_l·d and a multiple of 8. */
tp_status tp_attention_core(const void* qkv, int64_t ld_qkv, void* O,
                            int64_t b, int64_t s, int64_t H_l, int64_t d, int causal,
                            void* stream);

/* tp_attention_core_train -- tp_attention_core that also stores, for every
 * (sequence, local head, query), the base-2 log of the softmax normaliser,
 *     lse = log2 sum_k 2^(log2(e)·q·k/sqrt d)   over the visible keys k,
 * as f32 [b][H_l][s] (what the backward needs to recompute the softmax). */
tp_status tp_attention_core_train(const void* qkv, int64_t ld_qkv, void* O, float* lse,
                                  int64_t b, int64_t s, int64_t H_l, int64_t d, int causal,
                                  void* stream);

/* tp_attention_core_backward -- gradients of tp_attention_core
 * ([Megatron explainer] §3.2, backward; per head, with P the softmax of
 * S = Q·K^T/sqrt d): dV = P^T·dO, dP = dO·V^T, dS = P ⊙ (dP - rowsum(dO ⊙ O)),
 * dQ = dS·K/sqrt d, dK = dS^T·Q/sqrt d.
 *   qkv [b·s, ld_qkv], O and dO [b·s, H_l·d] bf16 (layouts of tp_attention_core);
 *   lse from tp_attention_core_train;
 *   dqkv [b·s, 3·H_l·d] bf16: dQ, dK, dV in qkv's column layout;
 *   D_ws f32 scratch of b·H_l·s elements (receives rowsum(dO ⊙ O)).
 * Deterministic: no atomics; d must be 128. */
tp_status tp_attention_core_backward(const void* qkv, int64_t ld_qkv, const void* O,
                                     const void* dO, const float* lse, void* dqkv, float* D_ws,
                                     int64_t b, int64_t s, int64_t H_l, int64_t d, int causal,
                                     void* stream);

/* tp_layernorm -- y = (x - mean)/sqrt(var + eps)·gamma + beta over each row of
 * x [M,h] (population variance, f32 statistics), the block's nn.LayerNorm(h)
 * ([PyTorch TP tutorial] 3.3).  x in TP_F32 or TP_BF16; y is bf16 [M,h];
 * gamma/beta f32 [h] or NULL.  Needs h % 8 == 0 and h <= 32768. */
tp_status tp_layernorm(const void* x, int in, void* y, const void* gamma,
                       const void* beta, float eps, int64_t M, int64_t h, void* stream);

/* ========================================================================
 * The vocabulary ends of the model, vocab-parallel ([Megatron explainer] §4).
 * The table E [V, h] (bf16) is split by rows: rank r holds E_r = rows
 * [vocab_start, vocab_start + V_r).  Token ids are int32 (4-byte aligned).
 * ====================================================================== */

/* tp_vocab_embedding_shard -- §4.1: out[m] = E_r[tokens[m] - vocab_start] for a
 * token in the rank's range, a zero row for any other token; summing the
 * ranks' outputs (tp_partial_sum, the all-reduce) gives the full lookup.
 *   out [M, h] in dtype out_dtype (TP_F32 or TP_BF16).  h % 8 == 0, V_r % 8 == 0. */
tp_status tp_vocab_embedding_shard(const int32_t* tokens, int64_t M, const void* E_r,
                                   int64_t V_r, int64_t h, int64_t vocab_start, void* out,
                                   int out_dtype, void* stream);

/* tp_vocab_ce_shard -- §4.2, one rank's local part of the cross-entropy with
 * the output layer tied to the input embedding: logits = H·E_r^T [M, V_r]
 * (never stored), and per token row, in the stable form (the row maximum
 * first; the page's exp-sum over raw logits overflows):
 *   stats[0..M)    m_r = max over the rank's logits,
 *   stats[M..2M)   s_r = sum exp(logit - m_r),
 *   stats[2M..3M)  t_r = the target's logit if the target is in the rank's
 *                  range, else 0.
 *   H [M, h] bf16, targets [M] int32, stats f32 [3·M];
 *   ws >= tp_vocab_ce_shard_workspace(M, V_r) bytes (statistics per row and 128-column piece).
 * h % 8 == 0, V_r % 8 == 0. */
size_t tp_vocab_ce_shard_workspace(int64_t M, int64_t V_r);
tp_status tp_vocab_ce_shard(const void* H, const void* E_r, const int32_t* targets, int64_t M,
                            int64_t h, int64_t V_r, int64_t vocab_start, float* stats, void* ws,
                            size_t ws_bytes, void* stream);

/* tp_vocab_ce_combine -- the all-reduces of §4.2 and the loss: from P ranks'
 * stats (rank r's [3·M] at stats + 3·M·r): m = max_r m_r,
 * s = sum_r s_r·exp(m_r - m), t = sum_r t_r, and per token
 *   loss[m] = log(s) + m - t   (= -log softmax(logits)[target]);
 * loss_mean (one float, or NULL) receives the mean over the M tokens.  Every
 * sum is taken in a fixed order. */
tp_status tp_vocab_ce_combine(const float* stats, int P, int64_t M, float* loss,
                              float* loss_mean, void* stream);

/* tp_vocab_parallel_ce -- all P ranks of the vocab-parallel cross-entropy on
 * this GPU: rank r's table E[r] (a HOST array of P device pointers) covers
 * vocabulary rows [r·V_r, (r+1)·V_r); the ranks' logits run as one grouped
 * launch (they share H), then each rank's statistics and the combine as
 * above.  ws >= tp_vocab_parallel_ce_workspace(M, V_r, P) bytes. */
size_t tp_vocab_parallel_ce_workspace(int64_t M, int64_t V_r, int P);
tp_status tp_vocab_parallel_ce(const void* H, const void* const* E, int P,
                               const int32_t* targets, int64_t M, int64_t h, int64_t V_r,
                               float* loss, float* loss_mean, void* ws, size_t ws_bytes,
                               void* stream);

/* ========================================================================
 * Measurement support (not part of the method).
 * ====================================================================== */

/* tp_block_shard_timed -- tp_block_shard (same arguments, same launches,
 * same results) that also records two HIP events (hipEvent_t handles, created
 * by the caller with timing enabled) on `stream`: ev_begin immediately before
 * and ev_end immediately after the launch of the MLP's column-parallel GEMM
 * with GeLU over all ranks, the block's dominant kernel.  hipEventElapsedTime
 * between them is that kernel's duration inside the step, as the benchmark
 * reports it.  Both events must be non-NULL (TP_ERR_NULL otherwise). */
tp_status tp_block_shard_timed(const void* x, void* out, int out_dtype, void* x1,
                               const void* ln1_g, const void* ln1_b,
                               const void* ln2_g, const void* ln2_b, float eps,
                               const void* const* W_qkv, const void* const* W_o,
                               const void* const* A, const void* const* B, int P,
                               void* ws, size_t ws_bytes, int64_t b, int64_t s, int64_t h,
                               int64_t H, int64_t d, int64_t F, void* stream,
                               void* ev_begin, void* ev_end);

/* tp_probe_mfma -- a register-only loop of MFMA 16x16x32 bf16 instructions:
 * `blocks` workgroups of 8 waves (two per SIMD), each wave issuing
 * 32 * iters independent MFMAs on values held in registers; nothing is loaded
 * from memory.  Each MFMA is 2*16*16*32 = 16384 FLOP, so a launch does
 * blocks * 8 * 32 * iters * 16384 FLOP.  Timed by the caller, it gives the
 * matrix-core throughput the GPU sustains under its current clock and power
 * limits -- the practical ceiling for any MFMA-bound kernel.
 *   out  device f32 buffer of blocks * 512 elements (receives the sums that
 *        keep the loop from being removed; the values mean nothing). */
tp_status tp_probe_mfma(float* out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TP_H */
