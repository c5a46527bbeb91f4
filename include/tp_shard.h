/*
 * tp_shard.h — C ABI of one GPU's share of a Megatron-style tensor-parallel transformer layer,
 * built for AMD MI355X (gfx950).
 *
 * The operations are those of "Megatron-LM: Training Multi-Billion Parameter Language Models
 * Using Model Parallelism" (paper digest), §3.4 Detailed, Sentence-Based Technical Breakdown,
 * and of "Tensor and pipeline parallelism, and choosing a layout" (ML Systems, lesson 9), §3,
 * Proposition (Megatron MLP split). Each call computes ONE rank's share from the replicated
 * input and that rank's own weight shard, and returns a sharded output or a full-size partial.
 * Summing partials across ranks (the paper's g in the forward pass and f in the backward pass)
 * is the caller's job; tp_sum_partials does it on one device.
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library never allocates
 *    device memory, frees or synchronises with the host, and keeps no state between calls
 *    apart from the thread-local error text: it creates no streams or events and takes no locks.
 *    Every kernel of a call is launched on the stream it is given (0 = null stream), in order, so
 *    calls on distinct streams are independent and a call can be captured into a graph.
 *  - Row-major, contiguous, 16-byte aligned. Tokens are rows: token = batch*s + position.
 *  - dt selects the element type of activations, weights, saved tensors and partials
 *    (TP_BF16: bfloat16 in, fp32 accumulate, bfloat16 out; TP_F32: fp32 throughout).
 *    Statistics (LayerNorm mean/rstd, attention lse, cross-entropy max/sumexp/target) are fp32.
 *  - Feature sizes (h, ffn/t, 3h/t, h/t, V/t) must be multiples of 8. Token counts are free.
 *  - Errors: arguments are checked on the host before any launch. On failure the call returns
 *    a non-zero tp_status, launches nothing, writes nothing and sets tp_last_error(). A launch
 *    failure reported by the HIP runtime returns TP_ERR_HIP. Forward calls with zero tokens
 *    return TP_OK and launch nothing; backward calls with zero tokens still write their weight
 *    and bias gradients (zeros, or unchanged when accumulating). Nothing aborts or throws
 *    across this boundary. Each bf16 or fp8 GEMM operand must be smaller than 2032 MiB
 *    (TP_ERR_UNSUPPORTED otherwise, before anything is launched).
 *  - Determinism: fixed reduction orders, no floating-point atomics; repeated calls on the
 *    same inputs give identical bits.
 *  - Workspace: calls that need scratch memory take (ws, ws_bytes); the matching *_workspace
 *    function returns the minimum size for the same shape arguments. The library does not keep
 *    anything in the workspace between calls.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t only */

#ifdef __cplusplus
extern "C" {
#endif

#define TP_ABI_VERSION 2

typedef enum tp_status {
    TP_OK = 0,
    TP_ERR_ARG = 1,         /* null pointer, t < 1, r outside [0, t), bad flag */
    TP_ERR_SHAPE = 2,       /* a size is negative, not divisible as required, or not a multiple of 8 */
    TP_ERR_DTYPE = 3,       /* unknown dtype */
    TP_ERR_WORKSPACE = 4,   /* ws_bytes smaller than the *_workspace query returns */
    TP_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
    TP_ERR_UNSUPPORTED = 6  /* valid request the library does not implement (e.g. fp32 attention) */
} tp_status;

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Dropout of one site. Passage: "Megatron-LM ..." digest §3.4, "Random Number Generation
 * Handling": residual dropout after g must draw the same pattern on every rank (pass the same seed
 * and stream on all ranks), attention dropout a different one per rank (pass a per-rank stream).
 * Generator (the pages name none): Philox4x32-10 (Salmon et al., SC 2011) with key = seed
 * (low word first) and counter = (call low, call high, 0, stream). One call gives eight 16-bit
 * uniforms u[j] = 16-bit half j%2 (low first) of word j/2; an element is kept iff u >= thr with
 * thr = round(p * 65536), and kept values are scaled by 65536 / (65536 - thr).
 * Residual sites over a [rows, n] tensor: element (row, c) is slot c % 8 of call row * n/8 + c/8.
 * Attention: element (sequence b, global head hg, query q, key k), with `heads` heads in all and
 * n32 = ceil(s / 32), is slot ((k % 16) / 8) * 4 + k % 4 of call
 * ((((b * heads + hg) * s + q) * n32 + k / 32) * 2 + (k % 8) / 4) * 2 + (k % 32) / 16.
 * A NULL tp_dropout pointer, or p = 0, means no dropout.
 * Attention sites also need `mask`: device memory of tp_attn_dropout_mask_bytes() bytes, laid out
 * as [b][heads/t][s][ceil(s/32)] 32-bit words whose bit j keeps key 32*kt + j of word (.., q, kt).
 * tp_attn_shard_fwd writes it; tp_attn_shard_bwd reads it (same p; seed and stream unused). */
typedef struct tp_dropout {
    float p;            /* drop probability, [0, 1) */
    uint32_t stream;    /* counter word 3 */
    uint64_t seed;      /* Philox key */
    uint32_t* mask;     /* attention only: keep bits, written by the forward, read by the backward */
} tp_dropout;

/* Version of this header's ABI (TP_ABI_VERSION). */
int tp_abi_version(void);

/* Text of the last error on the calling thread; "" if the last call succeeded. The pointer is
 * valid until the next tp_* call on the same thread. */
const char* tp_last_error(void);

/* ---------------------------------------------------------------------------------------------
 * MLP block, column-parallel first GEMM + row-parallel second GEMM.
 * Passage: "Megatron-LM ..." digest §3.4, "Column-Parallel GEMM for the First MLP Layer"
 * (A cut by columns, GeLU applied locally) and "Row-Parallel GEMM for the Second MLP Layer"
 * (B cut by rows, each rank's product is a full-size partial summed by g). GeLU is the erf form
 * ("Megatron-LM, annotated", §2.2).
 *
 * Rank r of t, F_t = ffn/t:
 *   X    [T, h]    replicated input (f is the identity forward)
 *   A_r  [h, F_t]  columns r*F_t .. (r+1)*F_t of A [h, ffn]
 *   b1_r [F_t]     the same slice of the first bias (may be NULL: no bias)
 *   B_r  [F_t, h]  rows r*F_t .. (r+1)*F_t of B [ffn, h]
 * Outputs (saved for backward):
 *   U_r  [T, F_t]  X A_r + b1_r          (pre-activation)
 *   Y_r  [T, F_t]  GeLU(U_r)
 *   Z_r  [T, h]    Y_r B_r, the rank's partial WITHOUT the second bias (added once after the sum)
 * ------------------------------------------------------------------------------------------- */
tp_status tp_mlp_shard_fwd(int T, int h, int ffn, int t, int r, tp_dtype dt,
                           const void* X, const void* A_r, const void* b1_r, const void* B_r,
                           void* U_r, void* Y_r, void* Z_r, hipStream_t stream);

/* Backward of the MLP shard. Passage: "Tensor and pipeline parallelism ..." §3, Proposition
 * (Megatron MLP split), proof steps 4-5:
 *   dU_r = (G B_r^T) * GeLU'(U_r)   (kept in the workspace)
 *   dB_r = Y_r^T G     [F_t, h]      dA_r = X^T dU_r  [h, F_t]    db1_r = column sums of dU_r [F_t]
 *   dX_r = dU_r A_r^T  [T, h]        the rank's partial of dL/dX; f sums the ranks' partials.
 * G [T, h] = dL/dZ is replicated (g is the identity backward). db1_r may be NULL.
 * accumulate = 0 overwrites dA_r, db1_r, dB_r; 1 adds into them (dX_r is always overwritten). */
size_t tp_mlp_shard_bwd_workspace(int T, int h, int ffn, int t, tp_dtype dt);
tp_status tp_mlp_shard_bwd(int T, int h, int ffn, int t, int r, tp_dtype dt,
                           const void* X, const void* A_r, const void* B_r, const void* U_r,
                           const void* Y_r, const void* G, void* dX_r, void* dA_r, void* db1_r,
                           void* dB_r, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Self-attention block, head-sharded. Passage: "Megatron-LM ..." digest §3.4, "Attention Head
 * Parallelism in the Self-Attention Block" (Q, K, V cut by columns along whole heads; softmax
 * of query key^T / sqrt(d_k) times value per head, locally; output projection cut by rows,
 * partials summed by g). Causal masking: a GPT-2 decoder attends left to right
 * ("Megatron-LM, annotated", §2.2). Only dt = TP_BF16 is implemented (fp32 softmax inside).
 *
 * Rank r of t owns heads r*heads/t .. (r+1)*heads/t - 1; d = h/heads; h_t = h/t:
 *   Xn     [b*s, h]     replicated (normalised) input
 *   Wqkv_r [h, 3h_t]    [Wq[:, H_r] | Wk[:, H_r] | Wv[:, H_r]] with H_r the rank's head columns
 *   bqkv_r [3h_t]       the matching bias slices (may be NULL)
 *   Wo_r   [h_t, h]     rows H_r of the output projection
 * Outputs (saved for backward):
 *   QKV_r  [b*s, 3h_t]  Xn Wqkv_r + bqkv_r, packed [Q | K | V], local head j at columns j*d
 *   O_r    [b*s, h_t]   attention output of the rank's heads
 *   lse_r  [b, heads/t, s] fp32, natural log of each query's softmax denominator
 *   Z_r    [b*s, h]     O_r Wo_r, partial WITHOUT the output bias
 * causal = 1: query i sees keys j <= i of its own sequence; 0: all keys of the sequence. */
tp_status tp_attn_shard_fwd(int b, int s, int h, int heads, int t, int r, tp_dtype dt, int causal,
                            const void* Xn, const void* Wqkv_r, const void* bqkv_r, const void* Wo_r,
                            void* QKV_r, void* O_r, float* lse_r, void* Z_r, const tp_dropout* drop,
                            hipStream_t stream);

/* Bytes of the keep-bit mask of one attention dropout site (tp_dropout.mask), for rank shapes
 * b, s and heads/t heads. */
size_t tp_attn_dropout_mask_bytes(int b, int s, int heads, int t);

/* Backward of the attention shard for G [b*s, h] = dL/dZ (replicated). The attention chain is the
 * textbook one (not on the pages): dO = G Wo_r^T; D = rowsum(dO * O); P recomputed from lse;
 * dV = P^T dO; dS = P * (dO V^T - D); dQ = dS K / sqrt(d); dK = dS^T Q / sqrt(d).
 * Outputs: dXn_r [b*s, h] partial (f sums them); dWqkv_r [h, 3h_t]; dbqkv_r [3h_t] (may be NULL);
 * dWo_r [h_t, h]. accumulate as in tp_mlp_shard_bwd (dXn_r always overwritten).
 * With the forward's attention dropout (drop with the same p and the mask it wrote): dV = P~^T dO
 * and dS = P * ((dO V^T) * keep * scale - D), P~ = P * keep * scale; D = rowsum(dO * O) holds as
 * is because O = P~ V.
 * The workspace holds dO, D, dQKV, split-K partials and dS in bf16 (b * heads/t * ceil(s/64)^2
 * blocks of 64 x 64; the dK/dV pass writes it, the dQ pass reads it). */
size_t tp_attn_shard_bwd_workspace(int b, int s, int h, int heads, int t, tp_dtype dt);
tp_status tp_attn_shard_bwd(int b, int s, int h, int heads, int t, int r, tp_dtype dt, int causal,
                            const void* Xn, const void* Wqkv_r, const void* Wo_r, const void* QKV_r,
                            const void* O_r, const float* lse_r, const void* G, void* dXn_r,
                            void* dWqkv_r, void* dbqkv_r, void* dWo_r, int accumulate,
                            const tp_dropout* drop, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Vocabulary-parallel fused logits GEMM + cross-entropy statistics. Passage: "Megatron-LM ..."
 * digest §3.4, "Output Embedding Parallelism and the Fused Cross-Entropy Optimization" (logits
 * X E_r^T on the rank's vocabulary rows; per-rank maximum; sums of exponentials; the correct
 * token's logit; padding so each rank's share is a multiple of 128; weight tying).
 * The logits never reach memory. Rank r owns global columns [r*V_t, (r+1)*V_t), V_t = Vpad/t.
 *   X [N, h]; E_r [V_t, h] rows of the tied embedding; targets int32 [N] in [0, Vreal)
 *   (targets are not range-checked: that would need a device sync; out-of-range ids give 0).
 * Outputs per token (fp32 / int32, [N] each):
 *   max_r     maximum logit over the rank's columns
 *   sumexp_r  sum of exp(logit - max_r) over the rank's columns
 *   tgt_r     the target's logit if this rank owns it, else 0
 *   argmax_r  global column index of max_r, lowest index on ties (may be NULL)
 * mask_padding = 1 treats columns >= Vreal as -inf; 0 scores them like any other column.
 * dt = TP_BF16 only. */
size_t tp_vocab_xent_shard_fwd_workspace(int N, int h, int Vpad, int t, tp_dtype dt);
tp_status tp_vocab_xent_shard_fwd(int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt,
                                  int mask_padding, const void* X, const void* E_r,
                                  const int32_t* targets, float* max_r, float* sumexp_r, float* tgt_r,
                                  int32_t* argmax_r, void* ws, size_t ws_bytes, hipStream_t stream);

/* tp_vocab_xent_shard_fwd without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results, with the per-(tile, token) partials in a library-owned scratch array of
 * TP_XENT_NOALLOC_SCRATCH_BYTES per device (allocated with the library's code object on a device's
 * first use, held until the process ends). The call itself allocates nothing. A shape whose
 * partials need more (tp_vocab_xent_shard_fwd_workspace bytes) is refused with
 * TP_ERR_UNSUPPORTED before any launch: 8 MiB holds e.g. N = 8192 tokens at V_t = 6400 (3.7 MB)
 * and up to ~18,000 tokens at that V_t. Every call on a device shares that device's array, which
 * keeps the last call's contents; calls that overlap in time on one device (on different streams
 * or host threads) race on it and must be serialised by the caller. */
#define TP_XENT_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
size_t tp_vocab_xent_shard_fwd_noalloc_max_bytes(void);
tp_status tp_vocab_xent_shard_fwd_noalloc(int N, int h, int Vpad, int Vreal, int t, int r,
                                          tp_dtype dt, int mask_padding, const void* X,
                                          const void* E_r, const int32_t* targets, float* max_r,
                                          float* sumexp_r, float* tgt_r, int32_t* argmax_r,
                                          hipStream_t stream);

/* The rank's fp32 logits [N, V_t], stored. For verification of the fused statistics; not on the
 * hot path. It runs the same bf16 MFMA main loop as tp_vocab_xent_shard_fwd but with the
 * library's ordinary tile plan for the shape, not the fused call's tiles. Every tile shape sums
 * each logit over k in the same order (64-deep K tiles in increasing k, the same MFMA
 * instruction and k-steps inside a tile, no K split), so the stored logits carry exactly the
 * bits the fused epilogue reduces. */
tp_status tp_vocab_logits_shard(int N, int h, int Vpad, int t, int r, tp_dtype dt, const void* X,
                                const void* E_r, float* logits, hipStream_t stream);

/* The same per-token statistics as tp_vocab_xent_shard_fwd (max, sum of exponentials relative to
 * it, target logit, argmax as a global index), computed from the rank's materialised fp32 logits
 * [N, ld] (row n = token n, column v = the rank's vocabulary row v, as tp_vocab_logits_shard writes
 * them): the unfused form that the pages contrast the fused call with ("Megatron-LM ..." digest
 * §3.4, output embedding parallelism: gathering the b*s*v logits instead of b*s scalars). A pass
 * over HBM: N * V_t * 4 bytes read, 16 bytes per token written. Max, argmax (lowest column on ties)
 * and target logit are exact functions of the logits; the sum of exponentials is summed in its own
 * order (within fp32 rounding of the fused call's). mask_padding as for the fused call.
 * ld >= V_t, ld % 4 == 0; argmax_r may be NULL. */
tp_status tp_vocab_xent_stats_from_logits(int N, int Vpad, int Vreal, int t, int r, int mask_padding,
                                          const float* logits, int ld, const int32_t* targets,
                                          float* max_r, float* sumexp_r, float* tgt_r, int32_t* argmax_r,
                                          hipStream_t stream);

/* Merge of t ranks' statistics into per-token losses, standing in for the cross-entropy's
 * all-reduces on one device: M = max_r max_r; S = sum_r sumexp_r exp(max_r - M);
 * loss = M + log S - sum_r tgt_r. max_r/sumexp_r/tgt_r are HOST arrays of t device pointers.
 * loss [N] fp32; mean_loss (1 float, may be NULL) gets the mean over N; max_all and sumexp_all
 * ([N] fp32, may be NULL) receive M and S, the merged statistics the backward needs. */
tp_status tp_vocab_xent_combine(int N, int t, const float* const* max_r, const float* const* sumexp_r,
                                const float* const* tgt_r, float* loss, float* mean_loss,
                                float* max_all, float* sumexp_all, hipStream_t stream);

/* Backward of the vocabulary-parallel cross-entropy for rank r (the pages give the forward,
 * "Megatron-LM ..." digest §3.4 steps 1-6; the gradient is the textbook derivative of the same
 * loss). With the merged per-token statistics M = max_all and S = sumexp_all (from
 * tp_vocab_xent_combine) and the upstream gradient dloss ([N] fp32; 1/N each for the mean loss):
 *   dlogits[n, v] = dloss[n] * (exp(y[n, v] - M[n]) / S[n] - [r*V_t + v == targets[n]])
 * over the rank's columns (0 on padding columns when mask_padding = 1), y = X E_r^T recomputed
 * (the logits are never kept), and
 *   dX_r [N, h]  = dlogits E_r    a full-size partial: the sum over ranks is dL/dX (the f point)
 *   dE_r [V_t, h] (+)= dlogits^T X   rank r's rows of dL/dE (accumulate = 1 adds, for the tied
 *                                    input embedding's share)
 * X, E_r, dX_r, dE_r in bf16 (dt = TP_BF16 only), row-major. The workspace holds dlogits twice in
 * bf16 (vocabulary-major and token-major, 2 x V_t x N elements, the token count rounded up to 8
 * in the first). N = 0 writes zeros into dE_r (or leaves it unchanged when accumulating). */
size_t tp_vocab_xent_shard_bwd_workspace(int N, int h, int Vpad, int t, tp_dtype dt);
tp_status tp_vocab_xent_shard_bwd(int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt,
                                  int mask_padding, const void* X, const void* E_r,
                                  const int32_t* targets, const float* max_all,
                                  const float* sumexp_all, const float* dloss, void* dX_r, void* dE_r,
                                  int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Helpers for the replicated parts of the layer ("Megatron-LM ..." digest §3.4, "Duplicate
 * Computation vs. Communication": norm, dropout and residual are computed by every rank).
 * ------------------------------------------------------------------------------------------- */

/* out = residual + D(sum_{r=0}^{t-1} parts[r] + bias (broadcast over rows)), summed in fp32 in
 * rank order; D is the residual dropout of `drop` (a residual site over [rows, cols]) or the
 * identity when drop is NULL. parts is a HOST array of t device pointers to [rows, cols] tensors
 * of in_dt; bias [cols] and residual [rows, cols] are in out_dt and may be NULL. Stands in for g
 * (forward) and f (backward) on one device. */
tp_status tp_sum_partials(int rows, int cols, int t, tp_dtype in_dt, const void* const* parts,
                          const void* bias, const void* residual, void* out, tp_dtype out_dt,
                          const tp_dropout* drop, hipStream_t stream);

/* Fused consumer of the forward g in a pre-LN block ("Megatron-LM, annotated", §2.2; the layer
 * norm is replicated on every rank): out = residual + D(sum_{r=0}^{t-1} parts[r] + bias), summed
 * in fp32 in rank order and stored in dt (D: the residual dropout of `drop`, a residual site over
 * [T, h], or the identity when drop is NULL), then y = LayerNorm(out) exactly as tp_layernorm_fwd
 * would compute it from the stored out. parts is a HOST array of t device pointers to [T, h]
 * tensors; every tensor (parts, bias [h], residual [T, h], out, gamma, beta, y) is in dt; bias and
 * residual may be NULL; mean, rstd [T] fp32 may be NULL. h <= 8192. */
tp_status tp_sum_partials_layernorm(int T, int h, int t, tp_dtype dt, const void* const* parts,
                                    const void* bias, const void* residual, void* out, float eps,
                                    const void* gamma, const void* beta, void* y, float* mean,
                                    float* rstd, const tp_dropout* drop, hipStream_t stream);

/* y = D(x) for a residual dropout site over x, y [rows, cols] in dt (in place allowed): the
 * backward of the forward's dropout is the same mask and scale applied to the gradient.
 * drop must not be NULL (p = 0 copies). */
tp_status tp_dropout_apply(int rows, int cols, tp_dtype dt, const void* x, void* y,
                           const tp_dropout* drop, hipStream_t stream);

/* tp_dropout_apply fused with the column sums of its result: y = D(x) and colsum_out [cols] (+)=
 * sum over rows of y (fp32 sums of the values before rounding to dt, fixed order). In the backward
 * of a residual site this is the branch gradient together with the bias gradient of the
 * row-parallel layer that feeds the site. Workspace: tp_colsum_workspace(rows, cols, dt). */
tp_status tp_dropout_colsum(int rows, int cols, tp_dtype dt, const void* x, void* y,
                            const tp_dropout* drop, void* colsum_out, int accumulate, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Vocabulary-parallel input embedding. Passage: "Megatron-LM ..." digest §3.4, "Input Embedding
 * Parallelism": the table E [Vpad, h] is split over vocabulary entries; rank r holds
 * E_r = rows r*Vpad/t .. (r+1)*Vpad/t - 1 and returns, for each token, its row when the id falls
 * in that range and a zero row otherwise; g sums the ranks' partials into E[ids] on every rank.
 * ids: int32 [N] (ids outside [0, Vpad) give zero rows on every rank; the host does not read ids).
 * ------------------------------------------------------------------------------------------- */
tp_status tp_embedding_shard_fwd(int N, int h, int Vpad, int t, int r, tp_dtype dt,
                                 const int32_t* ids, const void* E_r, void* out, hipStream_t stream);

/* Backward of the lookup (the derivative of a gather; not on the pages): dE_r[v] (+)= sum of dX[i]
 * over the tokens i with ids[i] = r*Vpad/t + v, in increasing token order (a stable counting sort
 * in the workspace, then ordered fp32 sums: deterministic). dX [N, h] is the replicated gradient
 * of the summed embedding output. accumulate = 0 overwrites dE_r (rows without tokens become 0);
 * 1 adds into it (e.g. onto the output-embedding gradient of a tied table). */
size_t tp_embedding_shard_bwd_workspace(int N, int Vpad, int t);
tp_status tp_embedding_shard_bwd(int N, int h, int Vpad, int t, int r, tp_dtype dt,
                                 const int32_t* ids, const void* dX, void* dE_r, int accumulate,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* LayerNorm over the last dimension: y = (x - mean) / sqrt(var + eps) * gamma + beta with the
 * biased variance. x, y [T, h] and gamma, beta [h] in dt; mean, rstd [T] fp32 (may be NULL). */
tp_status tp_layernorm_fwd(int T, int h, tp_dtype dt, float eps, const void* x, const void* gamma,
                           const void* beta, void* y, float* mean, float* rstd, hipStream_t stream);

/* LayerNorm backward: dx = dres + d(LN)/dx^T dy; dgamma = sum_rows dy * xhat; dbeta = sum_rows dy.
 * dres [T, h] (the residual branch's gradient) may be NULL. dgamma/dbeta [h] in dt may be NULL.
 * Optional column sums taken in the same pass, [h] in dt, may be NULL: dres_colsum = sum_rows dres
 * (needs dres), dx_colsum = sum_rows dx (of dx before rounding to dt). Around a pre-LN block these
 * are the replicated bias gradients of the row-parallel layers: with dres the gradient of the
 * layer output and dy the summed MLP input gradient, dres_colsum is the MLP output bias's gradient
 * and dx_colsum the attention output bias's ("Megatron-LM, annotated", §3.5).
 * accumulate (0 or 1) applies to every [h] output, as above. The workspace holds four fp32
 * partial rows per block; tp_layernorm_bwd_workspace gives its size (0 when T = 0). */
size_t tp_layernorm_bwd_workspace(int T, int h, tp_dtype dt);
tp_status tp_layernorm_bwd(int T, int h, tp_dtype dt, const void* x, const void* gamma,
                           const float* mean, const float* rstd, const void* dy, const void* dres,
                           void* dx, void* dgamma, void* dbeta, void* dres_colsum, void* dx_colsum,
                           int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* Column sums of G [T, n] into out [n] (the replicated bias gradients of the row-parallel
 * layers), in a fixed order. */
size_t tp_colsum_workspace(int T, int n, tp_dtype dt);
tp_status tp_colsum(int T, int n, tp_dtype dt, const void* G, void* out, int accumulate,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * The bf16 GEMM the shard calls are built from, exposed on its own: the column-parallel linear
 * layer (replicated input times the rank's column block, bias and GeLU fused) and the
 * row-parallel one (sharded input times the rank's row block, a full-size partial) of
 * "Megatron-LM ..." digest §3.4, and their input and weight gradients ("Tensor and pipeline
 * parallelism ..." §3, Proposition proof steps 4-5), as one call each.
 *   P[M, N] = sum_k A(m, k) B(k, n), bf16 operands, fp32 accumulation, then the epilogue `epi`
 *   (tp_epilogue) into bf16 C [M, ldc] (and C2 for TP_EPI_BIAS_GELU).
 * Operand layouts: a_mn = 0: A(m, k) = A[m * lda + k] (K-contiguous); a_mn = 1:
 * A(m, k) = A[k * lda + m] (MN-contiguous); likewise b_mn for B(k, n) = B[n * ldb + k] or
 * B[k * ldb + n]. Implemented: (a_mn, b_mn) = (0, 0) input gradients G W^T, (0, 1) forward
 * products X W, (1, 1) weight gradients X^T G; (1, 0) returns TP_ERR_UNSUPPORTED.
 * N % 8 == 0; lda, ldb, ldc multiples of 8 and at least the contiguous extent; every operand
 * below 2032 MiB. accumulate (0/1) only with TP_EPI_STORE; bias bf16 [N] or NULL (not with
 * TP_EPI_DGELU, whose aux is U [M, ldc]). ws: with TP_EPI_STORE and ws_bytes >=
 * tp_gemm_bf16_workspace(...) the call may split K (fp32 partials in ws, summed in a fixed
 * order); otherwise ws is unused and may be NULL. M, N or K = 0: C is written as the epilogue of
 * a zero product (K = 0), or nothing happens (M or N = 0). */
typedef enum tp_epilogue {
    TP_EPI_STORE = 0,      /* C = P (+ bias[n]) (+ C if accumulate) */
    TP_EPI_BIAS_GELU = 1,  /* C = P (+ bias[n]) (the pre-activation U), C2 = GeLU(C) (erf form) */
    TP_EPI_DGELU = 2       /* C = P * GeLU'(aux[m, n]) (aux = U, row stride ldc) */
} tp_epilogue;

size_t tp_gemm_bf16_workspace(int M, int N, int K);
tp_status tp_gemm_bf16(int M, int N, int K, const void* A, int lda, int a_mn, const void* B, int ldb,
                       int b_mn, int epi, void* C, void* C2, int ldc, const void* bias, const void* aux,
                       int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * fp8 GEMMs for the layer shard (8-bit E4M3 operands, fp32 accumulation, bf16 outputs).
 * The pages train in 16-bit floating point with dynamic loss scaling ("Megatron-LM, annotated",
 * §4.2 Training optimization and hyperparameters) and define no 8-bit format; the scheme here is
 * this library's own. Format: OCP E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * largest finite 448; 0x7F/0xFF are NaN; no infinities).
 * ------------------------------------------------------------------------------------------- */
/* Per-tensor quantisation of x [rows, cols] (row stride ldx, dt = TP_BF16 or TP_F32):
 *   amax = max |x|; e = the largest integer with amax * 2^e <= 448 (0 when amax is 0 or not
 *   finite), clamped to [-126, 126]; code = E4M3(x * 2^e), round to nearest even, saturating
 *   at +-448 (x * 2^e is exact, so this is the only rounding); *descale = 2^-e.
 * Outputs (device memory): codes [rows, ldc] (row layout) and/or codes_t [cols, ldt] (the
 * transpose, for GEMMs whose reduction runs over x's rows); either may be NULL, not both.
 * amax (one float) may be NULL; descale (one float) is required. The workspace holds the amax
 * partials. NaN inputs are outside the contract (the max ignores them). cols % 8 == 0,
 * ldx % 8 == 0, ldc and ldt multiples of 16. rows or cols = 0 writes descale = 1 (and amax = 0). */
size_t tp_fp8_quantize_workspace(int rows, int cols);
tp_status tp_fp8_quantize(int rows, int cols, tp_dtype dt, const void* x, int ldx, uint8_t* codes,
                          int ldc, uint8_t* codes_t, int ldt, float* amax, float* descale,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* P[M, N] = (*a_descale) * (*b_descale) * sum_k dec(A[m, k]) * dec(B[n, k]) with A [M, lda] and
 * B [N, ldb] E4M3 code matrices, both K-contiguous (row strides in bytes), fp32 accumulation,
 * then the epilogue `epi` (tp_epilogue) into bf16 C [M, ldc] (and C2 for TP_EPI_BIAS_GELU).
 * The descales are device pointers to one float each, normally those tp_fp8_quantize wrote.
 * In the layer: X A_r is A = codes of X, B = codes_t of A_r; the input gradient G W^T is
 * A = codes of G, B = codes of W; a weight gradient X^T G is A = codes_t of X, B = codes_t of G.
 * K % 16 == 0, lda and ldb multiples of 16 and >= K, N % 8 == 0, ldc % 8 == 0 and >= N.
 * accumulate (0/1) only with TP_EPI_STORE; bias is bf16 [N] or NULL (not with TP_EPI_DGELU).
 * ws: with TP_EPI_STORE and ws_bytes >= tp_gemm_fp8_workspace(M, N, K), the call may split K
 * (fp32 partials in ws, summed in a fixed order); otherwise ws is unused and may be NULL. */
size_t tp_gemm_fp8_workspace(int M, int N, int K);
tp_status tp_gemm_fp8(int M, int N, int K, const uint8_t* A, int lda, const float* a_descale,
                      const uint8_t* B, int ldb, const float* b_descale, int epi, void* C, void* C2,
                      int ldc, const void* bias, const void* aux, int accumulate, void* ws,
                      size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TP_SHARD_H */
