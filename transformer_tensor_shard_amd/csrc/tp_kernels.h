// Internal launcher declarations shared by the HIP translation units of
// libtp.so.  Not part of the public ABI (include/tp.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

// Operand layouts of the bf16 GEMM (row-major storage, leading dimensions in
// elements): NN  A [M,K], B [K,N];  NT  A [M,K], B [N,K] (C = A·B^T);
// TN  A [K,M], B [K,N] (C = A^T·B).
enum GemmLayout { GEMM_NN = 0, GEMM_NT = 1, GEMM_TN = 2 };
// Epilogues: v = acc + bias;  NONE  C = v;  GELU  C = GeLU(v);
// GELU_BWD  C = v · GeLU'(aux) (aux: the saved bf16 pre-activation);
// DUAL  C = bf16 GeLU(v) and aux = bf16 v (the training forward).
// CE_STATS (the vocab-parallel cross-entropy's logits, NT, f32): no C is
// written; for every output row and 128-column piece j of the row, C[g] (as
// float*) receives at [(row·ceil(N/128) + j)·2] the piece's maximum m and
// sum_i exp(logit_i - m), computed the same way whatever the output-tile
// width; aux[g] (as float*) receives logit[row][targets[row] - vstart[g]] at
// [row] when that column is in range (the caller zeroes it).
enum GemmEpi { EPI_NONE = 0, EPI_GELU = 1, EPI_GELU_BWD = 2, EPI_DUAL = 3, EPI_CE_STATS = 4 };

// Up to kMaxBatch independent GEMMs launched together: group g computes
// C[g] = epi(op(A[g])·op(B[g]) + bias[g]), an [M[g], N[g]] product with
// leading dimensions lda[g], ldb[g], ldc[g]; layout, epilogue, K and output
// type are common.  Used for the emulated ranks of a block (identical
// shapes) and for the weight gradients of a backward (different shapes).
constexpr int kMaxBatch = 32;
struct GemmBatch {
    const __bf16* A[kMaxBatch];
    const __bf16* B[kMaxBatch];
    const float* bias[kMaxBatch];
    void* C[kMaxBatch];
    __bf16* aux[kMaxBatch];   // GELU_BWD: read, DUAL: written; [M,N] with ldaux
    int M[kMaxBatch], N[kMaxBatch];
    int64_t lda[kMaxBatch], ldb[kMaxBatch], ldc[kMaxBatch];
    const int* targets;       // CE_STATS: target token id per row
    int vstart[kMaxBatch];    // CE_STATS: first vocab id of group g's columns
    int count;
    int band;       // set by the launcher: tile order for groups sharing A
    int causal_k;   // A is zero past its diagonal (A[m][k] = 0 for k > m, NN layout): a
                    // tile's K loop stops after its last row (only zero terms are dropped)
    // Split of the last, partly filled wave of workgroups (f32 output, no
    // epilogue): the caller offers split_ws (split_ws_bytes of device memory
    // free for the launch); the launcher may then run every tile of workgroup
    // id >= split_from as split_ways workgroups over equal K ranges, range 0
    // writing C and range p >= 1 the BM x (tile width) f32 block p-1 of tile
    // (id - split_from) in split_ws, and adds those blocks to C in order p = 1,
    // 2, ... in a second launch (set by the launcher: split_from, split_ways,
    // split_tail = the number of tail workgroups).
    float* split_ws;
    int64_t split_ws_bytes;
    int split_from, split_ways, split_tail;
};
// Supported (layout, epilogue, output) combinations: NN with NONE / GELU
// (bf16 or f32) and DUAL (bf16); NT with NONE / GELU_BWD (bf16 or f32) and
// CE_STATS (f32); TN with NONE (bf16 or f32).  Others return hipErrorInvalidValue.  The caller checks
// shapes: M, N, K multiples of 8 along contiguous dimensions, leading
// dimensions multiples of 8.
hipError_t gemm_bf16_batched(const GemmBatch& batch, int layout, int epi, int64_t lda,
                             int64_t ldb, int64_t ldc, int64_t ldaux, int64_t M, int64_t N,
                             int64_t K, bool out_bf16, hipStream_t stream);
// Groups with their own M[g], N[g], lda[g], ldb[g], ldc[g] (filled by the
// caller; groups with M or N of 0 are skipped), common K.
hipError_t gemm_bf16_grouped(const GemmBatch& batch, int layout, int epi, int64_t ldaux,
                             int64_t K, bool out_bf16, hipStream_t stream);

// Attention with Q, K, V split along the feature dimension over P ranks
// (kv_split.hip): partial scores per rank, their sum and the softmax, then
// O = P·V.  (sequence, head) pairs run kKvChunk at a time; rows up to kKvMaxS.
constexpr int kKvChunk = 32;
constexpr int kKvMaxS = 8192;
// a chunk's O = P·V products run as one grouped GEMM launch
static_assert(kKvChunk <= kMaxBatch, "a K/V-split chunk must fit one grouped GEMM launch");
int64_t kv_split_workspace_bytes(int64_t pairs, int64_t s, int64_t d, int P);
hipError_t kv_split_attention(const __bf16* qkv, int64_t ld, __bf16* O, int64_t ldo, int b, int s,
                              int H, int d, int P, bool causal, void* ws, hipStream_t stream);
// The forward (NN) form: epilogue GELU or NONE.
hipError_t gemm_bf16_batched(const GemmBatch& batch, int64_t lda, int64_t ldb, int64_t ldc,
                             int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                             hipStream_t stream);

// C[M,N] = epi(A[M,K]·B[K,N] + bias) on bf16 inputs with the MFMA kernel.
// Shapes and alignment are validated by the caller (tp_abi.cpp).
hipError_t gemm_bf16(const void* A, int64_t lda, const void* B, int64_t ldb,
                     const float* bias, void* C, int64_t ldc,
                     int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                     hipStream_t stream);

// Same contract on f32 inputs (plain FMA kernel, used by the f32 path).
hipError_t gemm_f32(const float* A, int64_t lda, const float* B, int64_t ldb,
                    const float* bias, void* C, int64_t ldc,
                    int64_t M, int64_t N, int64_t K, bool out_bf16, bool gelu,
                    hipStream_t stream);

// Causal / full softmax(Q K^T / sqrt(d)) V for every (rank, sequence, local
// head); d == 128.  Rank r's qkv is [b*s, ld_qkv] bf16 at qkv + r*qkv_rank_stride,
// its O is [b*s, H_l*128] bf16 at O + r*o_rank_stride (strides in elements).
// If lse is not NULL it receives, per (rank, sequence, head, query), the log2
// softmax normaliser L = log2 sum_k 2^(s_k·log2(e)/sqrt(d)) as f32
// [ranks][b][H_l][s].
hipError_t attention_fwd(const void* qkv, int64_t ld_qkv, void* O,
                         int64_t b, int64_t s, int64_t H_l, bool causal,
                         hipStream_t stream, int ranks = 1, int64_t qkv_rank_stride = 0,
                         int64_t o_rank_stride = 0, float* lse = nullptr);

// Backward of attention_fwd for one rank: from qkv, O, the upstream gradient
// dO ([b*s, H_l*128] bf16, leading dimension H_l*128) and lse, writes
// dqkv [b*s, 3*H_l*128] bf16 (dQ, dK, dV in qkv's column layout) and
// D = rowsum(dO ⊙ O) into Dvec (f32 [b][H_l][s]).
hipError_t attention_bwd(const void* qkv, int64_t ld_qkv, const void* O, const void* dO,
                         const float* lse, float* Dvec, void* dqkv, int64_t b, int64_t s,
                         int64_t H_l, bool causal, hipStream_t stream);

// y = LayerNorm(x) rows of length h, y in bf16.
hipError_t layernorm(const void* x, bool x_bf16, void* y, const float* gamma,
                     const float* beta, float eps, int64_t M, int64_t h,
                     hipStream_t stream);

// Z = sum_r parts[r] (+bias[col]) (+residual).
hipError_t partial_sum(void* Z, bool out_bf16, const void* parts, bool parts_bf16, int P,
                       int64_t M, int64_t h, const float* bias,
                       const void* residual, bool res_bf16, hipStream_t stream);

// The same sum computed one row per workgroup (h % 4 == 0, h <= 16384); if
// ln_out is not NULL, also ln_out = LayerNorm(Z row) in bf16.
hipError_t row_sum(void* Z, bool out_bf16, const void* parts, bool parts_bf16, int P,
                   int64_t M, int64_t h, const float* bias, const void* residual, bool res_bf16,
                   void* ln_out, const float* gamma, const float* beta, float eps,
                   hipStream_t stream);

// out[n] = Σ_m X[m, n] for bf16 X [M, N] (N % 8 == 0, ldx % 8 == 0) in a
// fixed order: row chunks of kColSumRows summed into part [chunks, N] f32
// (chunks = col_sum_chunks(M) <= 65535), then the chunks in order.
constexpr int64_t kColSumRows = 256;
int64_t col_sum_chunks(int64_t M);
hipError_t col_sum(float* out, const void* X, int64_t ldx, int64_t M, int64_t N, float* part,
                   hipStream_t stream);

// Vocab-parallel ends.  embed_shard: out[m] = E_r[tokens[m] - vstart] when
// that row exists, else zeros (h % 8 == 0).  fill_zero: p[0..n) = 0.
// ce_rank_reduce: CE_STATS tile statistics [M][ntn][2] -> m_r (stats[0..M)),
// s_r (stats[M..2M)).  ce_combine: ranks' [3][M] statistics (rank r at
// stats + 3·M·r) -> loss [M]; if loss_mean is not NULL also its mean.
hipError_t embed_shard(const int* tokens, int64_t M, const void* E_r, int64_t V_r, int64_t h,
                       int64_t vstart, void* out, bool out_bf16, hipStream_t stream);
hipError_t fill_zero(float* p, int64_t n, hipStream_t stream);
hipError_t ce_rank_reduce(const float* tiles, int ntn, int64_t M, float* stats,
                          hipStream_t stream);
hipError_t ce_combine(const float* stats, int P, int64_t M, float* loss, float* loss_mean,
                      hipStream_t stream);

// Compute units of the current device (256 on MI355X; queried once per
// device), for launch-shape choices.
int cu_count();

// Output-tile width (192, 256 or 384 columns) that gemm_bf16_grouped /
// gemm_bf16_batched use for this launch on the current device.
int gemm_tile_cols(const GemmBatch& b, int layout, int epi, int64_t K);

// Register-only MFMA 16x16x32 bf16 loop: `blocks` workgroups of 8 waves, each
// wave issuing 32 * iters MFMAs; out receives blocks * 512 floats.
hipError_t mfma_probe(float* out, int blocks, int iters, hipStream_t stream);

}  // namespace tpk
