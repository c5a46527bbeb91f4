// Host-side interface between the translation units: GEMM requests, tile planning and the
// kernel launchers. Everything here is plain host C++; no torch types.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rng.h"

namespace tp {

enum EpiKind {
    EPI_STORE = 0,      // out = acc (+ bias[col]) (+ out if accumulate)
    EPI_BIAS_GELU = 1,  // out = acc + bias (pre-activation U), out2 = GeLU(U)
    EPI_DGELU = 2,      // out = acc * GeLU'(aux)
    EPI_STORE_T = 3,    // fp32 out[col*ldc + row] = acc (transposed store)
    EPI_XENT = 4,       // cross-entropy tile statistics (xent.h)
    EPI_XENT_GRAD = 5,  // cross-entropy logits gradient, stored vocab-major and token-major (xent.h)
};

// C[M,N] = sum_k A(m,k) B(k,n). a_mn / b_mn: operand is MN-contiguous (element (mn,k) at
// p[k*ld + mn]) instead of K-contiguous (p[mn*ld + k]).
struct GemmReq {
    int M, N, K;
    const void* A; int lda; int a_mn;
    const void* B; int ldb; int b_mn;
    int epi;
    void* out; void* out2; int ldc;
    const void* bias; const void* aux; int accumulate;
    // EPI_XENT, EPI_XENT_GRAD
    const int32_t* targets; int col0, Vreal, mask;
    int row0;   // EPI_XENT: added to the reported argmax rows (a launch over a slice of the rows)
    // EPI_XENT_GRAD: merged per-token max and sum, upstream gradient; out2 = token-major copy (ld2)
    const float* stat_m; const float* stat_s; const float* dloss; int ld2;
    // fp8 GEMM: device pointers to the per-tensor descales of A and B
    const float* descale_a; const float* descale_b;
    // EPI_DGELU (bf16): if set, column sums of the stored output, one row per BM-row tile
    // ([ceil(M / plan.bm)][N] floats)
    float* colpart;
    // bf16 GEMMs with split-K: an unrelated column-sum job run by the split-K reduction's launch,
    // cs_out (bf16 [cs_n]) (+)= sums over the cs_nb rows of cs_part [cs_nb][cs_n] (cs_n % 4 == 0).
    // Only for plans with splits > 1 (without splits there is no reduction launch to carry it).
    const float* cs_part; void* cs_out; int cs_nb, cs_n, cs_accumulate;
};

struct GemmPlan {
    int cfg;      // 0: 256x256 (8 waves), 1: 128x128 (4 waves), 2: 256x192 (8 waves),
                  // 3: 64x64 (4 waves, 4 LDS stages), 4: 128x128 (4 waves, 3 LDS stages); 3 and 4
                  // with both operands K-contiguous (otherwise the two-stage 128x128 runs)
    int splits;   // K splits (>1 only when the request allows it)
    int bm, bn;
};

// Pick a tile configuration and K split count for a bf16 GEMM. allow_split permits split-K
// with fp32 partials (only plain stores). Pure function of the shape.
GemmPlan plan_gemm_bf16(int M, int N, int K, bool allow_split);
size_t split_ws_bytes(const GemmPlan& p, int M, int N);

// Launch one bf16 GEMM (+ split-K reduction if the plan has splits). ws must hold
// split_ws_bytes(plan) bytes when plan.splits > 1.
hipError_t gemm_bf16(const GemmReq& r, const GemmPlan& plan, void* ws, hipStream_t st);
// Two independent GEMMs in one launch on 128x128 tiles: r1 with both operands K-contiguous and a
// plain store, r2 with both MN-contiguous, split splits2 ways over K (fp32 partials in ws2,
// split_ws_bytes bytes for that split count, reduced in split order after). plan_gemm_pair says
// whether the pair fits one round of two workgroups per CU with comparable work per unit (and
// gives splits2); otherwise the two run as ordinary GEMMs.
bool plan_gemm_pair(const GemmReq& r1, const GemmReq& r2, int& splits2);
hipError_t gemm_bf16_pair(const GemmReq& r1, const GemmReq& r2, int splits2, void* ws2, hipStream_t st);
// Launch one fp32 SIMT GEMM.
hipError_t gemm_f32(const GemmReq& r, hipStream_t st);

// fp8 (E4M3) GEMM, both operands K-contiguous code matrices (lda/ldb in bytes); epilogues
// EPI_STORE (split-K allowed), EPI_BIAS_GELU, EPI_DGELU with bf16 outputs.
GemmPlan plan_gemm_fp8(int M, int N, int K, bool allow_split);
hipError_t gemm_fp8(const GemmReq& r, const GemmPlan& plan, void* ws, hipStream_t st);
// Per-tensor E4M3 quantisation of x [rows, cols] (dt 0 fp32, 1 bf16): codes [rows, ldc] and/or
// codes_t [cols, ldt] (transposed), amax (optional) and descale = 2^-e, each one float.
size_t fp8_quantize_ws_bytes();
hipError_t fp8_quantize(int dt, int rows, int cols, const void* x, int ldx, uint8_t* codes, int ldc,
                        uint8_t* codes_t, int ldt, float* amax, float* descale, float* ws, hipStream_t st);

// Per-layout instantiations (separate translation units).
hipError_t gemm_bf16_nn(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st);   // A K-contig, B MN-contig
hipError_t gemm_bf16_nt(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st);   // both K-contig
hipError_t gemm_bf16_tn(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st);   // both MN-contig

// Attention (bf16, head width d)
// dp.thr = 0: no dropout; otherwise attention dropout with dp.mask written by attn_fwd, read by attn_bwd.
// attn_bwd's dSws holds the bf16 score gradients between its two passes: attn_bwd_ds_bytes(b, s, heads_t)
// bytes (every 64 x 64 block of every head; a causal mask uses a little over half). colpart (may be
// null): column sums of the stored dQKV per 64-token tile, [b * ceil(s/64)][3 h_t] floats.
hipError_t attn_fwd(int b, int s, int h_t, int heads_t, int d, int causal, const void* QKV, void* O, float* lse,
                    const DropParams& dp, hipStream_t st);
hipError_t attn_bwd(int b, int s, int h_t, int heads_t, int d, int causal, const void* QKV, const void* O,
                    const float* lse, const void* dO, float* Dws, void* dSws, void* dQKV, float* colpart,
                    const DropParams& dp, hipStream_t st);
size_t attn_bwd_ds_bytes(int b, int s, int heads_t);

// Fused logits GEMM of a vocabulary shard (Vt rows x N tokens, depth K), in two launches: 256x256
// tiles over rows [0, main_rows) -- as many whole rounds of tiles over the 256 CUs as the shape
// holds -- and 64x64 tiles (two workgroups per CU) over the remaining rows, so the last round
// is not a partly filled round of large tiles. When the shape has no whole round, or its tiles
// fill whole rounds, one launch with the ordinary plan covers all rows (main_rows = Vt).
// tiles_m = tile rows of both parts (the per-token partials the merge reads).
struct VocabPlan {
    int main_rows;
    GemmPlan main, tail;
    int tiles_m;
};
VocabPlan plan_vocab(int Vt, int N, int K);

// A GEMM whose tiles leave a partly filled last round: rows [0, main_rows) in whole rounds of the
// ordinary plan's tiles, rows [main_rows, M) in one round of small tiles (64x64 on four LDS stages
// when both operands are K-contiguous, else 128x128), two launches in row order. main_rows = M
// (one launch) when the ordinary plan fills whole rounds or the remainder does not fit one round.
struct RowSplitPlan {
    int main_rows;
    GemmPlan main, tail;
};
RowSplitPlan plan_row_split(int M, int N, int K, bool both_kcontig);

// Cross-entropy merge / combine
hipError_t xent_merge(const void* part, int tiles_m, int N, int col0, float* mx, float* se, float* tg,
                      int32_t* am, hipStream_t st);
// Per-token statistics (the fused call's outputs) from materialised fp32 logits [N][ld]
hipError_t xent_stats_from_logits(const float* logits, int ld, int N, int Vt, int col0, int Vreal, int mask,
                                  const int32_t* targets, float* mx, float* se, float* tg, int32_t* am,
                                  hipStream_t st);
hipError_t xent_combine(int N, int t, const float* const* mx, const float* const* se, const float* const* tg,
                        float* loss, float* mean, float* max_all, float* sumexp_all, hipStream_t st);

// Norm / elementwise (dt: 0 fp32, 1 bf16)
int ln_bwd_blocks(int rows);
hipError_t layernorm_fwd(int dt, int rows, int h, float eps, const void* x, const void* g, const void* b, void* y,
                         float* mean, float* rstd, hipStream_t st);
// out = residual + D(sum_r parts[r] + bias) (all dt; D = residual dropout, identity when
// drop.thr = 0), then y = LayerNorm(out as stored)
hipError_t sum_partials_layernorm(int dt, int rows, int h, int t, const void* const* parts, const void* bias,
                                  const void* residual, void* out, float eps, const void* g, const void* b, void* y,
                                  float* mean, float* rstd, const DropParams& drop, hipStream_t st);
// dres_sum / dx_sum: optional column sums of dres and of dx (the bias gradients of the row-parallel
// layers on either side of the residual branch)
hipError_t layernorm_bwd(int dt, int rows, int h, const void* x, const void* g, const float* mean,
                         const float* rstd, const void* dy, const void* dres, void* dx, void* dg, void* db,
                         void* dres_sum, void* dx_sum, int accumulate, float* ws, hipStream_t st);
int colsum_row_blocks(int rows);
hipError_t colsum(int dt, int rows, int n, const void* G, void* out, int accumulate, float* ws, hipStream_t st);
// out (+)= sum over the nb rows of part [nb][n] (n % 4 == 0), in a fixed order; nb = 0 gives zeros
hipError_t colsum_reduce(int dt, int nb, int n, const float* part, void* out, int accumulate, hipStream_t st);
hipError_t sum_partials(int in_dt, int out_dt, size_t rows, int cols, int t, const void* const* parts,
                        const void* bias, const void* residual, void* out, const DropParams& drop, hipStream_t st);
// y = D(x) over [rows, n] (n % 8 == 0, in place allowed) and out (+)= column sums of y (fp32
// partials in ws: colsum_row_blocks(rows) x n floats)
hipError_t dropout_colsum(int dt, int rows, int n, const void* x, void* y, const DropParams& dp, void* out,
                          int accumulate, float* ws, hipStream_t st);
// y = D(x) over n contiguous elements of a tensor whose row length is a multiple of 8
hipError_t dropout(int dt, size_t n, const void* x, void* y, const DropParams& drop, hipStream_t st);

// Vocabulary-parallel embedding (embedding.hip)
hipError_t embedding_fwd(int dt, int N, int h, int Vt, int r, const int32_t* ids, const void* E_r, void* out,
                         hipStream_t st);
size_t embedding_bwd_ws_bytes(int N, int Vt);
hipError_t embedding_bwd(int dt, int N, int h, int Vt, int r, const int32_t* ids, const void* dX, void* dE_r,
                         int accumulate, void* ws, hipStream_t st);

}  // namespace tp
