// C ABI entry points: host-side validation, workspace carving and launch sequencing.
// Operation definitions and argument conventions are documented in include/tp_shard.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <initializer_list>
#include <string>

#include "launch.h"
#include "tp_shard.h"

using namespace tp;

namespace {

thread_local std::string g_err;

tp_status fail(tp_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

tp_status ok() {
    g_err.clear();
    return TP_OK;
}

#define HIP_TRY(expr, what)                                                                          \
    do {                                                                                             \
        hipError_t e_ = (expr);                                                                      \
        if (e_ != hipSuccess) return fail(TP_ERR_HIP, "%s: %s", (what), hipGetErrorString(e_));      \
    } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// required pointer: non-null and 16-byte aligned
#define NEED(p)                                                                                      \
    do {                                                                                             \
        if (!(p)) return fail(TP_ERR_ARG, "%s: argument '%s' is NULL", fn, #p);                      \
        if (!aligned16(p)) return fail(TP_ERR_ARG, "%s: argument '%s' is not 16-byte aligned", fn, #p); \
    } while (0)
// optional pointer: null, or 16-byte aligned
#define OPT(p)                                                                                       \
    do {                                                                                             \
        if ((p) && !aligned16(p)) return fail(TP_ERR_ARG, "%s: argument '%s' is not 16-byte aligned", fn, #p); \
    } while (0)

tp_status check_dt(const char* fn, tp_dtype dt) {
    if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "%s: unknown dtype %d", fn, (int)dt);
    return TP_OK;
}

tp_status check_rank(const char* fn, int t, int r) {
    if (t < 1) return fail(TP_ERR_ARG, "%s: tp degree t=%d must be >= 1", fn, t);
    if (r < 0 || r >= t) return fail(TP_ERR_ARG, "%s: rank r=%d outside [0, %d)", fn, r, t);
    return TP_OK;
}

tp_status check_mult8(const char* fn, const char* what, long v) {
    if (v <= 0 || v % 8 != 0) return fail(TP_ERR_SHAPE, "%s: %s=%ld must be a positive multiple of 8", fn, what, v);
    return TP_OK;
}

size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// bf16 and fp8 GEMM operands are addressed with 32-bit buffer offsets, and chunks outside an
// operand are fetched at an offset of 2032 MiB, which must lie past its end: every operand must be
// smaller. Checked before anything is launched.
constexpr size_t kMaxOperandBytes = (size_t)2032 << 20;
tp_status check_operands(const char* fn, size_t elem_bytes, std::initializer_list<size_t> elems) {
    for (size_t n : elems)
        if (n * elem_bytes >= kMaxOperandBytes)
            return fail(TP_ERR_UNSUPPORTED, "%s: a GEMM operand of %zu bytes reaches the 2032 MiB limit", fn,
                        n * elem_bytes);
    return TP_OK;
}

// tp_dropout -> kernel parameters: thr = round(p * 65536), scale = 65536 / (65536 - thr). NULL or
// p = 0 gives thr = 0 (no dropout).
tp_status make_drop(const char* fn, const tp_dropout* d, DropParams& out) {
    memset(&out, 0, sizeof(out));
    out.scale = 1.0f;
    if (!d) return TP_OK;
    if (!(d->p >= 0.0f && d->p < 1.0f)) return fail(TP_ERR_ARG, "%s: dropout p=%g must be in [0, 1)", fn, (double)d->p);
    const uint32_t thr = (uint32_t)std::floor((double)d->p * 65536.0 + 0.5);
    if (thr >= 65536u) return fail(TP_ERR_ARG, "%s: dropout p=%g rounds to 1", fn, (double)d->p);
    out.thr = thr;
    out.scale = (float)(65536.0 / (65536.0 - thr));
    out.seed_lo = (uint32_t)d->seed;
    out.seed_hi = (uint32_t)(d->seed >> 32);
    out.stream = d->stream;
    out.mask = d->mask;
    return TP_OK;
}

// attention site: also the rank's head offset and the mask buffer
tp_status attn_drop(const char* fn, const tp_dropout* d, int heads, int heads_t, int r, DropParams& out) {
    tp_status s = make_drop(fn, d, out);
    if (s != TP_OK) return s;
    out.head0 = r * heads_t;
    out.heads = heads;
    if (out.thr && (!out.mask || ((uintptr_t)out.mask & 3u)))
        return fail(TP_ERR_ARG, "%s: attention dropout needs a 4-byte aligned mask buffer", fn);
    return TP_OK;
}
size_t esize(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }

GemmReq req(int M, int N, int K, const void* A, int lda, int a_mn, const void* B, int ldb, int b_mn, int epi,
            void* out, int ldc) {
    GemmReq g;
    memset(&g, 0, sizeof(g));
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_mn = a_mn;
    g.B = B; g.ldb = ldb; g.b_mn = b_mn;
    g.epi = epi; g.out = out; g.ldc = ldc;
    return g;
}

hipError_t run_gemm(tp_dtype dt, const GemmReq& g, bool allow_split, void* split_ws, hipStream_t st) {
    if (dt == TP_F32) return gemm_f32(g, st);
    GemmPlan p = plan_gemm_bf16(g.M, g.N, g.K, allow_split);
    return gemm_bf16(g, p, split_ws, st);
}

size_t wgrad_split_ws(tp_dtype dt, int M, int N, int K) {
    if (dt != TP_BF16) return 0;
    return split_ws_bytes(plan_gemm_bf16(M, N, K, true), M, N);
}

size_t colsum_ws(int T, int n) { return (size_t)colsum_row_blocks(T) * n * sizeof(float); }

// dU | dB split partials | dA split partials | db1 column-sum partials (separate: the three can
// be in use at once on the two streams)
struct MlpWs {
    size_t dU, partB, partA, col, total;
};
MlpWs mlp_ws(int T, int h, int Ft, tp_dtype dt) {
    MlpWs w;
    w.dU = al256((size_t)T * Ft * esize(dt));
    w.partB = al256(wgrad_split_ws(dt, Ft, h, T));
    w.partA = al256(wgrad_split_ws(dt, h, Ft, T));
    // db1 partials: the column-sum pass's row blocks, or one row per 64 or more tokens (the dU
    // GEMM's tile rows), whichever is larger
    w.col = al256(std::max(colsum_ws(T, Ft), (size_t)((T + 63) / 64) * Ft * sizeof(float)));
    w.total = w.dU + w.partB + w.partA + w.col;
    return w;
}

// dO | D | dQKV | dWo split partials | dWqkv split partials | dbqkv column-sum partials | dS blocks
struct AttnWs {
    size_t dO, D, dQKV, partWo, partWqkv, col, dS, total;
};
AttnWs attn_ws(int b, int s, int h, int heads_t, int h_t) {
    long T = (long)b * s;
    AttnWs w;
    w.dO = al256((size_t)T * h_t * 2);
    w.D = al256((size_t)b * heads_t * s * sizeof(float));
    w.dQKV = al256((size_t)T * 3 * h_t * 2);
    // dWo split partials: its own plan's, or those of the launch paired with the dO GEMM
    size_t pw = wgrad_split_ws(TP_BF16, h_t, h, (int)T);
    {
        GemmReq r1 = req((int)T, h_t, h, nullptr, h, 0, nullptr, h, 0, EPI_STORE, nullptr, h_t);
        GemmReq r2 = req(h_t, h, (int)T, nullptr, h_t, 1, nullptr, h, 1, EPI_STORE, nullptr, h);
        int s2;
        if (plan_gemm_pair(r1, r2, s2)) pw = std::max(pw, (size_t)s2 * h_t * h * sizeof(float));
    }
    w.partWo = al256(pw);
    w.partWqkv = al256(wgrad_split_ws(TP_BF16, h, 3 * h_t, (int)T));
    // dbqkv partials: one row per 64-token tile of each sequence (at least the column-sum pass's)
    w.col = al256(std::max(colsum_ws((int)T, 3 * h_t), (size_t)b * ((s + 63) / 64) * 3 * h_t * sizeof(float)));
    w.dS = al256(attn_bwd_ds_bytes(b, s, heads_t));
    w.total = w.dO + w.D + w.dQKV + w.partWo + w.partWqkv + w.col + w.dS;
    return w;
}

tp_status check_mlp(const char* fn, int T, int h, int ffn, int t, int r, tp_dtype dt) {
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if ((s = check_rank(fn, t, r)) != TP_OK) return s;
    if (T < 0) return fail(TP_ERR_SHAPE, "%s: T=%d is negative", fn, T);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (ffn <= 0 || ffn % t != 0) return fail(TP_ERR_SHAPE, "%s: ffn=%d must be a positive multiple of t=%d", fn, ffn, t);
    if ((s = check_mult8(fn, "ffn/t", ffn / t)) != TP_OK) return s;
    if (dt != TP_BF16) return TP_OK;   // the fp32 GEMM indexes with 64-bit offsets
    const size_t Tz = (size_t)T, hz = (size_t)h, Fz = (size_t)(ffn / t);
    return check_operands(fn, 2, {Tz * hz, Tz * Fz, hz * Fz});
}

tp_status check_attn(const char* fn, int b, int s, int h, int heads, int t, int r, tp_dtype dt, int causal) {
    tp_status st;
    if ((st = check_dt(fn, dt)) != TP_OK) return st;
    if (dt != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "%s: attention is implemented for bf16 only", fn);
    if ((st = check_rank(fn, t, r)) != TP_OK) return st;
    if (causal != 0 && causal != 1) return fail(TP_ERR_ARG, "%s: causal=%d must be 0 or 1", fn, causal);
    if (b < 0 || s < 0) return fail(TP_ERR_SHAPE, "%s: b=%d, s=%d must be >= 0", fn, b, s);
    if (b > 65535) return fail(TP_ERR_SHAPE, "%s: b=%d exceeds 65535", fn, b);
    if ((long)b * s > INT32_MAX / 4) return fail(TP_ERR_SHAPE, "%s: b*s too large", fn);
    if ((st = check_mult8(fn, "h", h)) != TP_OK) return st;
    if (heads <= 0 || heads % t != 0) return fail(TP_ERR_SHAPE, "%s: heads=%d must be a positive multiple of t=%d", fn, heads, t);
    if (h % heads != 0) return fail(TP_ERR_SHAPE, "%s: h=%d is not a multiple of heads=%d", fn, h, heads);
    int d = h / heads;
    if (d != 64 && d != 96 && d != 128 && d != 192)
        return fail(TP_ERR_UNSUPPORTED, "%s: head width %d (supported: 64, 96, 128, 192)", fn, d);
    const size_t Tz = (size_t)b * s, hz = (size_t)h, qz = (size_t)3 * (h / t);
    return check_operands(fn, 2, {Tz * hz, Tz * qz, hz * qz});
}

tp_status check_vocab(const char* fn, int N, int h, int Vpad, int t, int r, tp_dtype dt) {
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (dt != TP_BF16) return fail(TP_ERR_UNSUPPORTED, "%s: the vocabulary GEMM is implemented for bf16 only", fn);
    if ((s = check_rank(fn, t, r)) != TP_OK) return s;
    if (N < 0) return fail(TP_ERR_SHAPE, "%s: N=%d is negative", fn, N);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (Vpad <= 0 || Vpad % t != 0) return fail(TP_ERR_SHAPE, "%s: Vpad=%d must be a positive multiple of t=%d", fn, Vpad, t);
    if ((s = check_mult8(fn, "Vpad/t", Vpad / t)) != TP_OK) return s;
    return check_operands(fn, 2, {(size_t)N * h, (size_t)(Vpad / t) * h});
}

size_t xent_ws(int N, int h, int Vt) {
    return al256((size_t)plan_vocab(Vt, N, h).tiles_m * (size_t)N * 16);
}

}  // namespace

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------------------------------------
tp_status tp_mlp_shard_fwd(int T, int h, int ffn, int t, int r, tp_dtype dt, const void* X, const void* A_r,
                           const void* b1_r, const void* B_r, void* U_r, void* Y_r, void* Z_r, hipStream_t stream) {
    const char* fn = "tp_mlp_shard_fwd";
    tp_status s = check_mlp(fn, T, h, ffn, t, r, dt);
    if (s != TP_OK) return s;
    NEED(X); NEED(A_r); NEED(B_r); NEED(U_r); NEED(Y_r); NEED(Z_r); OPT(b1_r);
    if (T == 0) return ok();
    const int Ft = ffn / t;
    GemmReq g1 = req(T, Ft, h, X, h, 0, A_r, Ft, 1, EPI_BIAS_GELU, U_r, Ft);
    g1.out2 = Y_r;
    g1.bias = b1_r;
    HIP_TRY(run_gemm(dt, g1, false, nullptr, stream), "tp_mlp_shard_fwd: column-parallel GEMM");
    GemmReq g2 = req(T, h, Ft, Y_r, Ft, 0, B_r, h, 1, EPI_STORE, Z_r, h);
    HIP_TRY(run_gemm(dt, g2, false, nullptr, stream), "tp_mlp_shard_fwd: row-parallel GEMM");
    return ok();
}

size_t tp_mlp_shard_bwd_workspace(int T, int h, int ffn, int t, tp_dtype dt) {
    if (T < 0 || h <= 0 || t < 1 || ffn <= 0 || ffn % t) return 0;
    return mlp_ws(T, h, ffn / t, dt).total;
}

tp_status tp_mlp_shard_bwd(int T, int h, int ffn, int t, int r, tp_dtype dt, const void* X, const void* A_r,
                           const void* B_r, const void* U_r, const void* Y_r, const void* G, void* dX_r, void* dA_r,
                           void* db1_r, void* dB_r, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "tp_mlp_shard_bwd";
    tp_status s = check_mlp(fn, T, h, ffn, t, r, dt);
    if (s != TP_OK) return s;
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    NEED(X); NEED(A_r); NEED(B_r); NEED(U_r); NEED(Y_r); NEED(G); NEED(dX_r); NEED(dA_r); NEED(dB_r); OPT(db1_r);
    const int Ft = ffn / t;
    MlpWs w = mlp_ws(T, h, Ft, dt);
    if (ws_bytes < w.total) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, w.total);
    if (w.total > 0) NEED(ws);
    char* base = (char*)ws;
    void* dU = base;
    void* partB = base + w.dU;
    void* partA = base + w.dU + w.partB;
    float* colp = (float*)(base + w.dU + w.partB + w.partA);
    // dU = (G B_r^T) * GeLU'(U_r); in bf16 its epilogue also writes the column sums of dU per tile
    // row, which db1 = column sums of dU then adds up
    GemmReq g = req(T, Ft, h, G, h, 0, B_r, h, 0, EPI_DGELU, dU, Ft);
    g.aux = U_r;
    const bool fused_db1 = db1_r && dt == TP_BF16;
    if (fused_db1) g.colpart = colp;
    HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_mlp_shard_bwd: dU GEMM");
    // dB_r = Y_r^T G; db1 = the sum of dU's per-tile column sums, added by the dB GEMM's split-K
    // reduction launch when it has one, else by a launch of its own
    g = req(Ft, h, T, Y_r, Ft, 1, G, h, 1, EPI_STORE, dB_r, h);
    g.accumulate = accumulate;
    bool db1_done = !db1_r;
    if (fused_db1) {
        const int bm = plan_gemm_bf16(T, Ft, h, false).bm, nb = T > 0 ? (T + bm - 1) / bm : 0;
        if (T > 0 && plan_gemm_bf16(Ft, h, T, true).splits > 1) {
            g.cs_part = colp; g.cs_out = db1_r; g.cs_nb = nb; g.cs_n = Ft; g.cs_accumulate = accumulate;
            db1_done = true;
        } else {
            HIP_TRY(colsum_reduce(1, nb, Ft, colp, db1_r, accumulate, stream), "tp_mlp_shard_bwd: db1");
            db1_done = true;
        }
    }
    if (!db1_done) HIP_TRY(colsum(0, T, Ft, dU, db1_r, accumulate, colp, stream), "tp_mlp_shard_bwd: db1");
    HIP_TRY(run_gemm(dt, g, true, partB, stream), "tp_mlp_shard_bwd: dB GEMM");
    // dA_r = X^T dU
    g = req(h, Ft, T, X, h, 1, dU, Ft, 1, EPI_STORE, dA_r, Ft);
    g.accumulate = accumulate;
    HIP_TRY(run_gemm(dt, g, true, partA, stream), "tp_mlp_shard_bwd: dA GEMM");
    // dX_r = dU A_r^T
    g = req(T, h, Ft, dU, Ft, 0, A_r, Ft, 0, EPI_STORE, dX_r, h);
    HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_mlp_shard_bwd: dX GEMM");
    return ok();
}

// ------------------------------------------------------------------------------------------------
tp_status tp_attn_shard_fwd(int b, int s, int h, int heads, int t, int r, tp_dtype dt, int causal, const void* Xn,
                            const void* Wqkv_r, const void* bqkv_r, const void* Wo_r, void* QKV_r, void* O_r,
                            float* lse_r, void* Z_r, const tp_dropout* drop, hipStream_t stream) {
    const char* fn = "tp_attn_shard_fwd";
    tp_status st = check_attn(fn, b, s, h, heads, t, r, dt, causal);
    if (st != TP_OK) return st;
    NEED(Xn); NEED(Wqkv_r); NEED(Wo_r); NEED(QKV_r); NEED(O_r); NEED(lse_r); NEED(Z_r); OPT(bqkv_r);
    const int heads_t = heads / t, d = h / heads, h_t = heads_t * d;
    DropParams dp;
    if ((st = attn_drop(fn, drop, heads, heads_t, r, dp)) != TP_OK) return st;
    const int T = b * s;
    if (T == 0) return ok();
    GemmReq g = req(T, 3 * h_t, h, Xn, h, 0, Wqkv_r, 3 * h_t, 1, EPI_STORE, QKV_r, 3 * h_t);
    g.bias = bqkv_r;
    HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_attn_shard_fwd: QKV GEMM");
    HIP_TRY(attn_fwd(b, s, h_t, heads_t, d, causal, QKV_r, O_r, lse_r, dp, stream), "tp_attn_shard_fwd: attention");
    g = req(T, h, h_t, O_r, h_t, 0, Wo_r, h, 1, EPI_STORE, Z_r, h);
    HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_attn_shard_fwd: output projection");
    return ok();
}

size_t tp_attn_dropout_mask_bytes(int b, int s, int heads, int t) {
    if (b < 0 || s < 0 || heads <= 0 || t < 1 || heads % t) return 0;
    return (size_t)b * (heads / t) * s * ((s + 31) / 32) * sizeof(uint32_t);
}

size_t tp_attn_shard_bwd_workspace(int b, int s, int h, int heads, int t, tp_dtype dt) {
    (void)dt;
    if (b < 0 || s < 0 || h <= 0 || heads <= 0 || t < 1 || heads % t || h % heads) return 0;
    int heads_t = heads / t, h_t = heads_t * (h / heads);
    return attn_ws(b, s, h, heads_t, h_t).total;
}

tp_status tp_attn_shard_bwd(int b, int s, int h, int heads, int t, int r, tp_dtype dt, int causal, const void* Xn,
                            const void* Wqkv_r, const void* Wo_r, const void* QKV_r, const void* O_r,
                            const float* lse_r, const void* G, void* dXn_r, void* dWqkv_r, void* dbqkv_r,
                            void* dWo_r, int accumulate, const tp_dropout* drop, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    const char* fn = "tp_attn_shard_bwd";
    tp_status st = check_attn(fn, b, s, h, heads, t, r, dt, causal);
    if (st != TP_OK) return st;
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    NEED(Xn); NEED(Wqkv_r); NEED(Wo_r); NEED(QKV_r); NEED(O_r); NEED(lse_r); NEED(G); NEED(dXn_r); NEED(dWqkv_r);
    NEED(dWo_r); OPT(dbqkv_r);
    const int T = b * s;
    const int heads_t = heads / t, d = h / heads, h_t = heads_t * d;
    DropParams dp;
    if ((st = attn_drop(fn, drop, heads, heads_t, r, dp)) != TP_OK) return st;
    AttnWs w = attn_ws(b, s, h, heads_t, h_t);
    if (ws_bytes < w.total) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, w.total);
    if (w.total > 0) NEED(ws);
    char* base = (char*)ws;
    void* dO = base;
    float* Dv = (float*)(base + w.dO);
    void* dQKV = base + w.dO + w.D;
    void* partWo = base + w.dO + w.D + w.dQKV;
    void* partWqkv = base + w.dO + w.D + w.dQKV + w.partWo;
    float* colp = (float*)(base + w.dO + w.D + w.dQKV + w.partWo + w.partWqkv);
    void* dSw = base + w.dO + w.D + w.dQKV + w.partWo + w.partWqkv + w.col;
    // dO = G Wo_r^T and dWo_r = O_r^T G: independent, both thin (h/t columns or rows), so one
    // paired launch when they fit one round of the CUs together
    GemmReq g = req(T, h_t, h, G, h, 0, Wo_r, h, 0, EPI_STORE, dO, h_t);
    GemmReq gw = req(h_t, h, T, O_r, h_t, 1, G, h, 1, EPI_STORE, dWo_r, h);
    gw.accumulate = accumulate;
    int s2;
    if (plan_gemm_pair(g, gw, s2)) {
        HIP_TRY(gemm_bf16_pair(g, gw, s2, partWo, stream), "tp_attn_shard_bwd: dO + dWo GEMMs");
    } else {
        HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_attn_shard_bwd: dO GEMM");
        HIP_TRY(run_gemm(dt, gw, true, partWo, stream), "tp_attn_shard_bwd: dWo GEMM");
    }
    if (T > 0)
        HIP_TRY(attn_bwd(b, s, h_t, heads_t, d, causal, QKV_r, O_r, lse_r, dO, Dv, dSw, dQKV, dbqkv_r ? colp : nullptr,
                         dp, stream),
                "tp_attn_shard_bwd: attention backward");
    // dWqkv_r = Xn^T dQKV; dbqkv = the sum of the attention backward's per-tile column sums of dQKV,
    // added by the dWqkv GEMM's split-K reduction launch when it has one, else by a launch of its own
    g = req(h, 3 * h_t, T, Xn, h, 1, dQKV, 3 * h_t, 1, EPI_STORE, dWqkv_r, 3 * h_t);
    g.accumulate = accumulate;
    if (dbqkv_r) {
        const int nb = T > 0 ? b * ((s + 63) / 64) : 0;
        if (T > 0 && plan_gemm_bf16(h, 3 * h_t, T, true).splits > 1) {
            g.cs_part = colp; g.cs_out = dbqkv_r; g.cs_nb = nb; g.cs_n = 3 * h_t; g.cs_accumulate = accumulate;
        } else {
            HIP_TRY(colsum_reduce(1, nb, 3 * h_t, colp, dbqkv_r, accumulate, stream), "tp_attn_shard_bwd: dbqkv");
        }
    }
    HIP_TRY(run_gemm(dt, g, true, partWqkv, stream), "tp_attn_shard_bwd: dWqkv GEMM");
    // dXn_r = dQKV Wqkv_r^T
    g = req(T, h, 3 * h_t, dQKV, 3 * h_t, 0, Wqkv_r, 3 * h_t, 0, EPI_STORE, dXn_r, h);
    HIP_TRY(run_gemm(dt, g, false, nullptr, stream), "tp_attn_shard_bwd: dXn GEMM");
    return ok();
}

// ------------------------------------------------------------------------------------------------
size_t tp_vocab_xent_shard_fwd_workspace(int N, int h, int Vpad, int t, tp_dtype dt) {
    (void)dt;
    if (N < 0 || h <= 0 || t < 1 || Vpad <= 0 || Vpad % t) return 0;
    return xent_ws(N, h, Vpad / t);
}

// Argument checks shared by the two forms of the fused vocabulary call (workspace / library scratch).
static tp_status check_xent_fwd(const char* fn, int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt,
                                int mask_padding, const void* X, const void* E_r, const int32_t* targets, float* max_r,
                                float* sumexp_r, float* tgt_r, int32_t* argmax_r) {
    tp_status st = check_vocab(fn, N, h, Vpad, t, r, dt);
    if (st != TP_OK) return st;
    if (Vreal <= 0 || Vreal > Vpad) return fail(TP_ERR_SHAPE, "%s: Vreal=%d must be in [1, Vpad=%d]", fn, Vreal, Vpad);
    if (mask_padding != 0 && mask_padding != 1) return fail(TP_ERR_ARG, "%s: mask_padding=%d must be 0 or 1", fn, mask_padding);
    NEED(X); NEED(E_r); NEED(targets); NEED(max_r); NEED(sumexp_r); NEED(tgt_r); OPT(argmax_r);
    return TP_OK;
}

// The fused logits GEMM over rows [0, main_rows) and [main_rows, Vt) of the shard, then the tile
// merge; the tile partials go to `part` (xent_ws bytes). The tail's partials follow the main
// part's tile rows, so the merge reads the tiles in row order.
static tp_status launch_xent_fwd(const char* fn, int N, int h, int Vt, int Vreal, int r, int mask_padding,
                                 const void* X, const void* E_r, const int32_t* targets, float* max_r, float* sumexp_r,
                                 float* tgt_r, int32_t* argmax_r, void* part, hipStream_t stream) {
    const VocabPlan vp = plan_vocab(Vt, N, h);
    GemmReq g = req(vp.main_rows, N, h, E_r, h, 0, X, h, 0, EPI_XENT, part, 0);
    g.targets = targets;
    g.col0 = r * Vt;
    g.Vreal = Vreal;
    g.mask = mask_padding;
    HIP_TRY(gemm_bf16(g, vp.main, nullptr, stream), "tp_vocab_xent_shard_fwd: fused logits GEMM");
    if (vp.main_rows < Vt) {
        const int main_tiles = vp.main_rows / vp.main.bm;
        g.M = Vt - vp.main_rows;
        g.A = (const char*)E_r + (size_t)vp.main_rows * h * 2;
        g.out = (char*)part + (size_t)main_tiles * N * 16;
        g.col0 = r * Vt + vp.main_rows;
        g.row0 = vp.main_rows;
        HIP_TRY(gemm_bf16(g, vp.tail, nullptr, stream), "tp_vocab_xent_shard_fwd: fused logits GEMM (last rows)");
    }
    HIP_TRY(xent_merge(part, vp.tiles_m, N, r * Vt, max_r, sumexp_r, tgt_r, argmax_r, stream),
            "tp_vocab_xent_shard_fwd: tile merge");
    (void)fn;
    return ok();
}

tp_status tp_vocab_xent_shard_fwd(int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt, int mask_padding,
                                  const void* X, const void* E_r, const int32_t* targets, float* max_r,
                                  float* sumexp_r, float* tgt_r, int32_t* argmax_r, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
    const char* fn = "tp_vocab_xent_shard_fwd";
    tp_status st = check_xent_fwd(fn, N, h, Vpad, Vreal, t, r, dt, mask_padding, X, E_r, targets, max_r, sumexp_r,
                                  tgt_r, argmax_r);
    if (st != TP_OK) return st;
    const int Vt = Vpad / t;
    size_t need = xent_ws(N, h, Vt);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (need > 0) NEED(ws);
    if (N == 0) return ok();
    return launch_xent_fwd(fn, N, h, Vt, Vreal, r, mask_padding, X, E_r, targets, max_r, sumexp_r, tgt_r, argmax_r, ws,
                           stream);
}

}  // extern "C"

// Library-owned scratch for tp_vocab_xent_shard_fwd_noalloc: one copy per device, allocated with the
// code object when the library is first used on that device and kept until the process ends. Host
// code must not pass `tp_xent_scratch` itself to a kernel (in host code the name is a stand-in,
// not a device address): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char tp_xent_scratch[TP_XENT_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_xent_scratch[kMaxDevices];

// The current device's address of tp_xent_scratch (resolved on the first call on that device; a
// race between two first calls resolves the same address twice).
tp_status xent_scratch(const char* fn, void*& out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
    void* p = g_xent_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(tp_xent_scratch)), "hipGetSymbolAddress(tp_xent_scratch)");
        if (!p) return fail(TP_ERR_HIP, "%s: hipGetSymbolAddress returned NULL", fn);
        g_xent_scratch[dev].store(p, std::memory_order_release);
    }
    out = p;
    return TP_OK;
}
}  // namespace

extern "C" {

size_t tp_vocab_xent_shard_fwd_noalloc_max_bytes(void) { return TP_XENT_NOALLOC_SCRATCH_BYTES; }

tp_status tp_vocab_xent_shard_fwd_noalloc(int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt,
                                          int mask_padding, const void* X, const void* E_r, const int32_t* targets,
                                          float* max_r, float* sumexp_r, float* tgt_r, int32_t* argmax_r,
                                          hipStream_t stream) {
    const char* fn = "tp_vocab_xent_shard_fwd_noalloc";
    tp_status st = check_xent_fwd(fn, N, h, Vpad, Vreal, t, r, dt, mask_padding, X, E_r, targets, max_r, sumexp_r,
                                  tgt_r, argmax_r);
    if (st != TP_OK) return st;
    const int Vt = Vpad / t;
    const size_t need = xent_ws(N, h, Vt);
    if (need > TP_XENT_NOALLOC_SCRATCH_BYTES)
        return fail(TP_ERR_UNSUPPORTED, "%s: the tile partials need %zu bytes, beyond the %zu-byte scratch (use "
                    "tp_vocab_xent_shard_fwd with a workspace)", fn, need, (size_t)TP_XENT_NOALLOC_SCRATCH_BYTES);
    if (N == 0) return ok();
    void* part = nullptr;
    if ((st = xent_scratch(fn, part)) != TP_OK) return st;
    // every partial the merge reads is written by the GEMM of this call: nothing needs clearing
    return launch_xent_fwd(fn, N, h, Vt, Vreal, r, mask_padding, X, E_r, targets, max_r, sumexp_r, tgt_r, argmax_r,
                           part, stream);
}

tp_status tp_vocab_logits_shard(int N, int h, int Vpad, int t, int r, tp_dtype dt, const void* X, const void* E_r,
                                float* logits, hipStream_t stream) {
    const char* fn = "tp_vocab_logits_shard";
    tp_status st = check_vocab(fn, N, h, Vpad, t, r, dt);
    if (st != TP_OK) return st;
    NEED(X); NEED(E_r); NEED(logits);
    if (N == 0) return ok();
    const int Vt = Vpad / t;
    GemmPlan p = plan_gemm_bf16(Vt, N, h, false);
    GemmReq g = req(Vt, N, h, E_r, h, 0, X, h, 0, EPI_STORE_T, logits, Vt);
    HIP_TRY(gemm_bf16(g, p, nullptr, stream), "tp_vocab_logits_shard: logits GEMM");
    return ok();
}

tp_status tp_vocab_xent_stats_from_logits(int N, int Vpad, int Vreal, int t, int r, int mask_padding,
                                          const float* logits, int ld, const int32_t* targets, float* max_r,
                                          float* sumexp_r, float* tgt_r, int32_t* argmax_r, hipStream_t stream) {
    const char* fn = "tp_vocab_xent_stats_from_logits";
    tp_status st;
    if ((st = check_rank(fn, t, r)) != TP_OK) return st;
    if (N < 0) return fail(TP_ERR_SHAPE, "%s: N=%d is negative", fn, N);
    if (Vpad <= 0 || Vpad % t != 0) return fail(TP_ERR_SHAPE, "%s: Vpad=%d must be a positive multiple of t=%d", fn, Vpad, t);
    if ((st = check_mult8(fn, "Vpad/t", Vpad / t)) != TP_OK) return st;
    if (Vreal <= 0 || Vreal > Vpad) return fail(TP_ERR_SHAPE, "%s: Vreal=%d must be in [1, Vpad=%d]", fn, Vreal, Vpad);
    if (mask_padding != 0 && mask_padding != 1) return fail(TP_ERR_ARG, "%s: mask_padding=%d must be 0 or 1", fn, mask_padding);
    const int Vt = Vpad / t;
    if (ld < Vt || ld % 4 != 0) return fail(TP_ERR_SHAPE, "%s: ld=%d must be >= V_t=%d and a multiple of 4", fn, ld, Vt);
    NEED(logits); NEED(targets); NEED(max_r); NEED(sumexp_r); NEED(tgt_r); OPT(argmax_r);
    if (N == 0) return ok();
    HIP_TRY(xent_stats_from_logits(logits, ld, N, Vt, r * Vt, Vreal, mask_padding, targets, max_r, sumexp_r, tgt_r,
                                   argmax_r, stream), fn);
    return ok();
}

// dlogits copies: vocab-major [Vt][ldd] (ldd = N rounded up to 8) and token-major [N][Vt]
static size_t xent_bwd_ld(int N) { return ((size_t)N + 7) / 8 * 8; }
size_t tp_vocab_xent_shard_bwd_workspace(int N, int h, int Vpad, int t, tp_dtype dt) {
    (void)h; (void)dt;
    if (N < 0 || t < 1 || Vpad <= 0 || Vpad % t) return 0;
    const size_t Vt = (size_t)(Vpad / t);
    return al256(Vt * xent_bwd_ld(N) * 2) + al256((size_t)N * Vt * 2);
}

tp_status tp_vocab_xent_shard_bwd(int N, int h, int Vpad, int Vreal, int t, int r, tp_dtype dt, int mask_padding,
                                  const void* X, const void* E_r, const int32_t* targets, const float* max_all,
                                  const float* sumexp_all, const float* dloss, void* dX_r, void* dE_r, int accumulate,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "tp_vocab_xent_shard_bwd";
    tp_status st = check_vocab(fn, N, h, Vpad, t, r, dt);
    if (st != TP_OK) return st;
    if (Vreal <= 0 || Vreal > Vpad) return fail(TP_ERR_SHAPE, "%s: Vreal=%d must be in [1, Vpad=%d]", fn, Vreal, Vpad);
    if (mask_padding != 0 && mask_padding != 1) return fail(TP_ERR_ARG, "%s: mask_padding=%d must be 0 or 1", fn, mask_padding);
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    NEED(X); NEED(E_r); NEED(targets); NEED(max_all); NEED(sumexp_all); NEED(dloss); NEED(dX_r); NEED(dE_r);
    const int Vt = Vpad / t;
    const size_t need = tp_vocab_xent_shard_bwd_workspace(N, h, Vpad, t, dt);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (need > 0) NEED(ws);
    const int ldd = (int)xent_bwd_ld(N);
    // the two copies of the logits gradient are GEMM operands too (steps 2 and 3)
    if ((st = check_operands(fn, 2, {(size_t)N * Vt, (size_t)Vt * ldd})) != TP_OK) return st;
    void* D = ws;
    void* DT = (char*)ws + al256((size_t)Vt * ldd * 2);
    GemmReq g;
    if (N > 0) {
        // 1. logits again (E_r X^T), their gradient in the epilogue, stored in both layouts; the
        //    forward's tiling: whole rounds of 256x256 tiles, the remaining vocabulary rows on 64x64
        const VocabPlan lp = plan_vocab(Vt, N, h);
        g = req(lp.main_rows, N, h, E_r, h, 0, X, h, 0, EPI_XENT_GRAD, D, ldd);
        g.out2 = DT; g.ld2 = Vt;
        g.targets = targets; g.col0 = r * Vt; g.Vreal = Vreal; g.mask = mask_padding;
        g.stat_m = max_all; g.stat_s = sumexp_all; g.dloss = dloss;
        HIP_TRY(gemm_bf16(g, lp.main, nullptr, stream), "tp_vocab_xent_shard_bwd: logits gradient");
        if (lp.main_rows < Vt) {
            g.M = Vt - lp.main_rows;
            g.A = (const char*)E_r + (size_t)lp.main_rows * h * 2;
            g.out = (char*)D + (size_t)lp.main_rows * ldd * 2;
            g.out2 = (char*)DT + (size_t)lp.main_rows * 2;
            g.col0 = r * Vt + lp.main_rows;
            HIP_TRY(gemm_bf16(g, lp.tail, nullptr, stream), "tp_vocab_xent_shard_bwd: logits gradient (last rows)");
        }
        // 2. dX_r = dlogits E_r   (token-major dlogits, E_r read MN-contiguous)
        g = req(N, h, Vt, DT, Vt, 0, E_r, h, 1, EPI_STORE, dX_r, h);
        HIP_TRY(gemm_bf16(g, plan_gemm_bf16(N, h, Vt, false), nullptr, stream), "tp_vocab_xent_shard_bwd: dX GEMM");
    }
    // 3. dE_r (+)= dlogits^T X   (vocab-major dlogits, X read MN-contiguous; with no tokens the
    //    K = 0 product writes zeros, or leaves dE_r unchanged when accumulating)
    const RowSplitPlan ep = plan_row_split(Vt, h, N, false);
    g = req(ep.main_rows, h, N, D, ldd, 0, X, h, 1, EPI_STORE, dE_r, h);
    g.accumulate = accumulate;
    HIP_TRY(gemm_bf16(g, ep.main, nullptr, stream), "tp_vocab_xent_shard_bwd: dE GEMM");
    if (ep.main_rows < Vt) {
        g.M = Vt - ep.main_rows;
        g.A = (const char*)D + (size_t)ep.main_rows * ldd * 2;
        g.out = (char*)dE_r + (size_t)ep.main_rows * h * 2;
        HIP_TRY(gemm_bf16(g, ep.tail, nullptr, stream), "tp_vocab_xent_shard_bwd: dE GEMM (last rows)");
    }
    return ok();
}

tp_status tp_vocab_xent_combine(int N, int t, const float* const* max_r, const float* const* sumexp_r,
                                const float* const* tgt_r, float* loss, float* mean_loss, float* max_all,
                                float* sumexp_all, hipStream_t stream) {
    const char* fn = "tp_vocab_xent_combine";
    if (t < 1 || t > 64) return fail(TP_ERR_ARG, "%s: t=%d must be in [1, 64]", fn, t);
    if (N < 0) return fail(TP_ERR_SHAPE, "%s: N=%d is negative", fn, N);
    if (!max_r || !sumexp_r || !tgt_r) return fail(TP_ERR_ARG, "%s: pointer arrays must not be NULL", fn);
    for (int i = 0; i < t; ++i)
        if (!max_r[i] || !sumexp_r[i] || !tgt_r[i]) return fail(TP_ERR_ARG, "%s: rank %d pointer is NULL", fn, i);
    NEED(loss);
    if (N == 0) return ok();
    OPT(max_all); OPT(sumexp_all);
    HIP_TRY(xent_combine(N, t, max_r, sumexp_r, tgt_r, loss, mean_loss, max_all, sumexp_all, stream),
            "tp_vocab_xent_combine");
    return ok();
}

// ------------------------------------------------------------------------------------------------
tp_status tp_sum_partials(int rows, int cols, int t, tp_dtype in_dt, const void* const* parts, const void* bias,
                          const void* residual, void* out, tp_dtype out_dt, const tp_dropout* drop,
                          hipStream_t stream) {
    const char* fn = "tp_sum_partials";
    tp_status s;
    if ((s = check_dt(fn, in_dt)) != TP_OK || (s = check_dt(fn, out_dt)) != TP_OK) return s;
    if (t < 1 || t > 64) return fail(TP_ERR_ARG, "%s: t=%d must be in [1, 64]", fn, t);
    if (rows < 0) return fail(TP_ERR_SHAPE, "%s: rows=%d is negative", fn, rows);
    if ((s = check_mult8(fn, "cols", cols)) != TP_OK) return s;
    if (!parts) return fail(TP_ERR_ARG, "%s: parts is NULL", fn);
    for (int i = 0; i < t; ++i) {
        if (!parts[i]) return fail(TP_ERR_ARG, "%s: parts[%d] is NULL", fn, i);
        if (!aligned16(parts[i])) return fail(TP_ERR_ARG, "%s: parts[%d] is not 16-byte aligned", fn, i);
    }
    NEED(out); OPT(bias); OPT(residual);
    DropParams dp;
    if ((s = make_drop(fn, drop, dp)) != TP_OK) return s;
    HIP_TRY(sum_partials(in_dt == TP_BF16, out_dt == TP_BF16, (size_t)rows, cols, t, parts, bias, residual, out, dp,
                         stream),
            "tp_sum_partials");
    return ok();
}

tp_status tp_sum_partials_layernorm(int T, int h, int t, tp_dtype dt, const void* const* parts, const void* bias,
                                    const void* residual, void* out, float eps, const void* gamma, const void* beta,
                                    void* y, float* mean, float* rstd, const tp_dropout* drop, hipStream_t stream) {
    const char* fn = "tp_sum_partials_layernorm";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (t < 1 || t > 64) return fail(TP_ERR_ARG, "%s: t=%d must be in [1, 64]", fn, t);
    if (T < 0) return fail(TP_ERR_SHAPE, "%s: T=%d is negative", fn, T);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (h > 8192) return fail(TP_ERR_UNSUPPORTED, "%s: h=%d exceeds 8192", fn, h);
    if (!(eps >= 0.0f)) return fail(TP_ERR_ARG, "%s: eps must be >= 0", fn);
    if (!parts) return fail(TP_ERR_ARG, "%s: parts is NULL", fn);
    for (int i = 0; i < t; ++i) {
        if (!parts[i]) return fail(TP_ERR_ARG, "%s: parts[%d] is NULL", fn, i);
        if (!aligned16(parts[i])) return fail(TP_ERR_ARG, "%s: parts[%d] is not 16-byte aligned", fn, i);
    }
    NEED(out); OPT(bias); OPT(residual); NEED(gamma); NEED(beta); NEED(y); OPT(mean); OPT(rstd);
    DropParams dp;
    if ((s = make_drop(fn, drop, dp)) != TP_OK) return s;
    HIP_TRY(sum_partials_layernorm(dt == TP_BF16, T, h, t, parts, bias, residual, out, eps, gamma, beta, y, mean, rstd,
                                   dp, stream), fn);
    return ok();
}

tp_status tp_layernorm_fwd(int T, int h, tp_dtype dt, float eps, const void* x, const void* gamma, const void* beta,
                           void* y, float* mean, float* rstd, hipStream_t stream) {
    const char* fn = "tp_layernorm_fwd";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (T < 0) return fail(TP_ERR_SHAPE, "%s: T=%d is negative", fn, T);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (h > 8192) return fail(TP_ERR_UNSUPPORTED, "%s: h=%d exceeds 8192", fn, h);
    if (!(eps >= 0.0f)) return fail(TP_ERR_ARG, "%s: eps must be >= 0", fn);
    NEED(x); NEED(gamma); NEED(beta); NEED(y); OPT(mean); OPT(rstd);
    HIP_TRY(layernorm_fwd(dt == TP_BF16, T, h, eps, x, gamma, beta, y, mean, rstd, stream), fn);
    return ok();
}

size_t tp_layernorm_bwd_workspace(int T, int h, tp_dtype dt) {
    (void)dt;
    if (T <= 0 || h <= 0) return 0;
    return al256(4 * (size_t)ln_bwd_blocks(T) * h * sizeof(float));   // four column-sum partials
}

tp_status tp_layernorm_bwd(int T, int h, tp_dtype dt, const void* x, const void* gamma, const float* mean,
                           const float* rstd, const void* dy, const void* dres, void* dx, void* dgamma, void* dbeta,
                           void* dres_colsum, void* dx_colsum, int accumulate, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    const char* fn = "tp_layernorm_bwd";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (T < 0) return fail(TP_ERR_SHAPE, "%s: T=%d is negative", fn, T);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (h > 8192) return fail(TP_ERR_UNSUPPORTED, "%s: h=%d exceeds 8192", fn, h);
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    NEED(x); NEED(gamma); NEED(mean); NEED(rstd); NEED(dy); NEED(dx); OPT(dres); OPT(dgamma); OPT(dbeta);
    OPT(dres_colsum); OPT(dx_colsum);
    if (dres_colsum && !dres) return fail(TP_ERR_ARG, "%s: dres_colsum needs dres", fn);
    if (dgamma || dbeta || dres_colsum || dx_colsum) {
        size_t need = tp_layernorm_bwd_workspace(T, h, dt);
        if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
        if (need > 0) NEED(ws);
    }
    HIP_TRY(layernorm_bwd(dt == TP_BF16, T, h, x, gamma, mean, rstd, dy, dres, dx, dgamma, dbeta, dres_colsum,
                          dx_colsum, accumulate, (float*)ws, stream), fn);
    return ok();
}

size_t tp_colsum_workspace(int T, int n, tp_dtype dt) {
    (void)dt;
    if (T < 0 || n <= 0) return 0;
    return al256(colsum_ws(T, n));
}

tp_status tp_colsum(int T, int n, tp_dtype dt, const void* G, void* out, int accumulate, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
    const char* fn = "tp_colsum";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (T < 0) return fail(TP_ERR_SHAPE, "%s: T=%d is negative", fn, T);
    if ((s = check_mult8(fn, "n", n)) != TP_OK) return s;
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    NEED(G); NEED(out);
    size_t need = tp_colsum_workspace(T, n, dt);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (need > 0) NEED(ws);
    HIP_TRY(colsum(dt == TP_BF16, T, n, G, out, accumulate, (float*)ws, stream), fn);
    return ok();
}

/* ---- dropout and the vocabulary-parallel embedding ---- */

tp_status tp_dropout_apply(int rows, int cols, tp_dtype dt, const void* x, void* y, const tp_dropout* drop,
                           hipStream_t stream) {
    const char* fn = "tp_dropout_apply";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (rows < 0) return fail(TP_ERR_SHAPE, "%s: rows=%d is negative", fn, rows);
    if ((s = check_mult8(fn, "cols", cols)) != TP_OK) return s;
    if (!drop) return fail(TP_ERR_ARG, "%s: drop is NULL", fn);
    NEED(x); NEED(y);
    DropParams dp;
    if ((s = make_drop(fn, drop, dp)) != TP_OK) return s;
    const size_t n = (size_t)rows * cols;
    if (dp.thr == 0) {
        if (x != y) HIP_TRY(hipMemcpyAsync(y, x, n * esize(dt), hipMemcpyDeviceToDevice, stream), fn);
        return ok();
    }
    HIP_TRY(dropout(dt == TP_BF16, n, x, y, dp, stream), fn);
    return ok();
}

tp_status tp_dropout_colsum(int rows, int cols, tp_dtype dt, const void* x, void* y, const tp_dropout* drop,
                            void* colsum_out, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "tp_dropout_colsum";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (rows < 0) return fail(TP_ERR_SHAPE, "%s: rows=%d is negative", fn, rows);
    if ((s = check_mult8(fn, "cols", cols)) != TP_OK) return s;
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    if (!drop) return fail(TP_ERR_ARG, "%s: drop is NULL", fn);
    NEED(x); NEED(y); NEED(colsum_out);
    DropParams dp;
    if ((s = make_drop(fn, drop, dp)) != TP_OK) return s;
    const size_t need = tp_colsum_workspace(rows, cols, dt);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (need > 0) NEED(ws);
    HIP_TRY(dropout_colsum(dt == TP_BF16, rows, cols, x, y, dp, colsum_out, accumulate, (float*)ws, stream), fn);
    return ok();
}

tp_status tp_embedding_shard_fwd(int N, int h, int Vpad, int t, int r, tp_dtype dt, const int32_t* ids,
                                 const void* E_r, void* out, hipStream_t stream) {
    const char* fn = "tp_embedding_shard_fwd";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK || (s = check_rank(fn, t, r)) != TP_OK) return s;
    if (N < 0) return fail(TP_ERR_SHAPE, "%s: N=%d is negative", fn, N);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (Vpad <= 0 || Vpad % t != 0) return fail(TP_ERR_SHAPE, "%s: Vpad=%d must be a positive multiple of t", fn, Vpad);
    if ((long)N * h >= (1L << 31)) return fail(TP_ERR_SHAPE, "%s: N*h too large", fn);
    if (!ids) return fail(TP_ERR_ARG, "%s: ids is NULL", fn);
    NEED(E_r); NEED(out);
    HIP_TRY(embedding_fwd(dt == TP_BF16, N, h, Vpad / t, r, ids, E_r, out, stream), fn);
    return ok();
}

size_t tp_embedding_shard_bwd_workspace(int N, int Vpad, int t) {
    if (N < 0 || t < 1 || Vpad <= 0 || Vpad % t) return 0;
    return al256(embedding_bwd_ws_bytes(N, Vpad / t));
}

tp_status tp_embedding_shard_bwd(int N, int h, int Vpad, int t, int r, tp_dtype dt, const int32_t* ids,
                                 const void* dX, void* dE_r, int accumulate, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    const char* fn = "tp_embedding_shard_bwd";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK || (s = check_rank(fn, t, r)) != TP_OK) return s;
    if (N < 0) return fail(TP_ERR_SHAPE, "%s: N=%d is negative", fn, N);
    if ((s = check_mult8(fn, "h", h)) != TP_OK) return s;
    if (Vpad <= 0 || Vpad % t != 0) return fail(TP_ERR_SHAPE, "%s: Vpad=%d must be a positive multiple of t", fn, Vpad);
    if ((long)N * h >= (1L << 31)) return fail(TP_ERR_SHAPE, "%s: N*h too large", fn);
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    if (!ids && N > 0) return fail(TP_ERR_ARG, "%s: ids is NULL", fn);
    if (N > 0) NEED(dX);
    NEED(dE_r);
    size_t need = tp_embedding_shard_bwd_workspace(N, Vpad, t);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    NEED(ws);
    HIP_TRY(embedding_bwd(dt == TP_BF16, N, h, Vpad / t, r, ids, dX, dE_r, accumulate, ws, stream), fn);
    return ok();
}

/* ---- the bf16 GEMM on its own ---- */

size_t tp_gemm_bf16_workspace(int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return al256(split_ws_bytes(plan_gemm_bf16(M, N, K, true), M, N));
}

tp_status tp_gemm_bf16(int M, int N, int K, const void* A, int lda, int a_mn, const void* B, int ldb, int b_mn,
                       int epi, void* C, void* C2, int ldc, const void* bias, const void* aux, int accumulate,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "tp_gemm_bf16";
    if (M < 0 || N < 0 || K < 0) return fail(TP_ERR_SHAPE, "%s: M=%d N=%d K=%d must be >= 0", fn, M, N, K);
    if (N % 8 != 0) return fail(TP_ERR_SHAPE, "%s: N=%d must be a multiple of 8", fn, N);
    if ((a_mn != 0 && a_mn != 1) || (b_mn != 0 && b_mn != 1))
        return fail(TP_ERR_ARG, "%s: a_mn=%d, b_mn=%d must be 0 or 1", fn, a_mn, b_mn);
    if (a_mn && !b_mn) return fail(TP_ERR_UNSUPPORTED, "%s: A MN-contiguous with B K-contiguous", fn);
    const int a_ext = a_mn ? M : K, b_ext = b_mn ? N : K;
    if (lda < a_ext || lda % 8 != 0 || ldb < b_ext || ldb % 8 != 0)
        return fail(TP_ERR_SHAPE, "%s: lda=%d, ldb=%d must be multiples of 8 and >= %d, %d", fn, lda, ldb, a_ext, b_ext);
    if (ldc < N || ldc % 8 != 0) return fail(TP_ERR_SHAPE, "%s: ldc=%d must be >= N and a multiple of 8", fn, ldc);
    if (epi != TP_EPI_STORE && epi != TP_EPI_BIAS_GELU && epi != TP_EPI_DGELU)
        return fail(TP_ERR_ARG, "%s: unknown epilogue %d", fn, epi);
    // epilogues per layout: the forward products carry bias + GeLU, the input gradients GeLU'
    if ((epi == TP_EPI_BIAS_GELU && !(!a_mn && b_mn)) || (epi == TP_EPI_DGELU && !(!a_mn && !b_mn)))
        return fail(TP_ERR_UNSUPPORTED, "%s: epilogue %d with layout (a_mn=%d, b_mn=%d)", fn, epi, a_mn, b_mn);
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    if (accumulate && epi != TP_EPI_STORE) return fail(TP_ERR_ARG, "%s: accumulate needs TP_EPI_STORE", fn);
    NEED(A); NEED(B); NEED(C); OPT(bias);
    if (epi == TP_EPI_BIAS_GELU) NEED(C2);
    if (epi == TP_EPI_DGELU) {
        NEED(aux);
        if (bias) return fail(TP_ERR_ARG, "%s: TP_EPI_DGELU takes no bias", fn);
    }
    tp_status st = check_operands(fn, 2, {(size_t)(a_mn ? K : M) * lda, (size_t)(b_mn ? K : N) * ldb});
    if (st != TP_OK) return st;
    if (M == 0 || N == 0) return ok();
    const size_t need = tp_gemm_bf16_workspace(M, N, K);
    const bool split_ok = epi == TP_EPI_STORE && need > 0 && ws && aligned16(ws) && ws_bytes >= need;
    GemmReq g = req(M, N, K, A, lda, a_mn, B, ldb, b_mn,
                    epi == TP_EPI_STORE ? EPI_STORE : epi == TP_EPI_BIAS_GELU ? EPI_BIAS_GELU : EPI_DGELU, C, ldc);
    g.out2 = C2; g.bias = bias; g.aux = aux; g.accumulate = accumulate;
    HIP_TRY(gemm_bf16(g, plan_gemm_bf16(M, N, K, split_ok), split_ok ? ws : nullptr, stream), fn);
    return ok();
}

/* ---- fp8 (E4M3) quantisation and GEMM ---- */

size_t tp_fp8_quantize_workspace(int rows, int cols) {
    (void)rows; (void)cols;
    return al256(fp8_quantize_ws_bytes());
}

tp_status tp_fp8_quantize(int rows, int cols, tp_dtype dt, const void* x, int ldx, uint8_t* codes, int ldc,
                          uint8_t* codes_t, int ldt, float* amax, float* descale, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    const char* fn = "tp_fp8_quantize";
    tp_status s;
    if ((s = check_dt(fn, dt)) != TP_OK) return s;
    if (rows < 0 || cols < 0) return fail(TP_ERR_SHAPE, "%s: rows=%d cols=%d must be >= 0", fn, rows, cols);
    if (cols % 8 != 0) return fail(TP_ERR_SHAPE, "%s: cols=%d must be a multiple of 8", fn, cols);
    if ((long)rows * (cols / 8) >= (1L << 31)) return fail(TP_ERR_SHAPE, "%s: tensor too large", fn);
    if (ldx < cols || ldx % 8 != 0) return fail(TP_ERR_SHAPE, "%s: ldx=%d must be >= cols and a multiple of 8", fn, ldx);
    if (!codes && !codes_t) return fail(TP_ERR_ARG, "%s: codes and codes_t are both NULL", fn);
    NEED(x); OPT(codes); OPT(codes_t);
    if (codes && (ldc < cols || ldc % 16 != 0))
        return fail(TP_ERR_SHAPE, "%s: ldc=%d must be >= cols and a multiple of 16", fn, ldc);
    if (codes_t && (ldt < rows || ldt % 16 != 0))
        return fail(TP_ERR_SHAPE, "%s: ldt=%d must be >= rows and a multiple of 16", fn, ldt);
    if (!descale || ((uintptr_t)descale & 3u)) return fail(TP_ERR_ARG, "%s: descale is NULL or misaligned", fn);
    if (amax && ((uintptr_t)amax & 3u)) return fail(TP_ERR_ARG, "%s: amax is misaligned", fn);
    size_t need = tp_fp8_quantize_workspace(rows, cols);
    if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    NEED(ws);
    HIP_TRY(fp8_quantize(dt == TP_BF16, rows, cols, x, ldx, codes, ldc, codes_t, ldt, amax, descale, (float*)ws,
                         stream), fn);
    return ok();
}

size_t tp_gemm_fp8_workspace(int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return al256(split_ws_bytes(plan_gemm_fp8(M, N, K, true), M, N));
}

tp_status tp_gemm_fp8(int M, int N, int K, const uint8_t* A, int lda, const float* a_descale, const uint8_t* B,
                      int ldb, const float* b_descale, int epi, void* C, void* C2, int ldc, const void* bias,
                      const void* aux, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "tp_gemm_fp8";
    if (M < 0 || N < 0 || K < 0) return fail(TP_ERR_SHAPE, "%s: M=%d N=%d K=%d must be >= 0", fn, M, N, K);
    if (K % 16 != 0) return fail(TP_ERR_SHAPE, "%s: K=%d must be a multiple of 16", fn, K);
    if (N % 8 != 0) return fail(TP_ERR_SHAPE, "%s: N=%d must be a multiple of 8", fn, N);
    if (lda < K || lda % 16 != 0 || ldb < K || ldb % 16 != 0)
        return fail(TP_ERR_SHAPE, "%s: lda=%d, ldb=%d must be >= K and multiples of 16", fn, lda, ldb);
    if (ldc < N || ldc % 8 != 0) return fail(TP_ERR_SHAPE, "%s: ldc=%d must be >= N and a multiple of 8", fn, ldc);
    if (epi != TP_EPI_STORE && epi != TP_EPI_BIAS_GELU && epi != TP_EPI_DGELU)
        return fail(TP_ERR_ARG, "%s: unknown epilogue %d", fn, epi);
    if (accumulate != 0 && accumulate != 1) return fail(TP_ERR_ARG, "%s: accumulate=%d must be 0 or 1", fn, accumulate);
    if (accumulate && epi != TP_EPI_STORE) return fail(TP_ERR_ARG, "%s: accumulate needs TP_EPI_STORE", fn);
    NEED(A); NEED(B); NEED(C); OPT(bias);
    if (!a_descale || !b_descale || ((uintptr_t)a_descale & 3u) || ((uintptr_t)b_descale & 3u))
        return fail(TP_ERR_ARG, "%s: a_descale / b_descale NULL or misaligned", fn);
    if (epi == TP_EPI_BIAS_GELU) NEED(C2);
    if (epi == TP_EPI_DGELU) {
        NEED(aux);
        if (bias) return fail(TP_ERR_ARG, "%s: TP_EPI_DGELU takes no bias", fn);
    }
    tp_status st = check_operands(fn, 1, {(size_t)M * lda, (size_t)N * ldb});
    if (st != TP_OK) return st;
    if (M == 0 || N == 0) return ok();
    const size_t need = tp_gemm_fp8_workspace(M, N, K);
    const bool split_ok = epi == TP_EPI_STORE && ws && aligned16(ws) && ws_bytes >= need;
    GemmPlan p = plan_gemm_fp8(M, N, K, split_ok);
    GemmReq g = req(M, N, K, A, lda, 0, B, ldb, 0, epi, C, ldc);
    g.out2 = C2; g.bias = bias; g.aux = aux; g.accumulate = accumulate;
    g.descale_a = a_descale; g.descale_b = b_descale;
    HIP_TRY(gemm_fp8(g, p, split_ok ? ws : nullptr, stream), fn);
    return ok();
}

}  // extern "C"
