// Host-side tile planning for the bf16 MFMA GEMM and layout dispatch.
#include <hip/hip_runtime.h>
#include "launch.h"

namespace tp {

static const int kNCfg = 3;   // configurations the time model chooses among
// tile shape of every configuration (3: 64x64 four-stage, 4: 128x128 three-stage; both need
// K-contiguous operands and are picked only by plans below)
static const int kBM[5] = {256, 128, 256, 64, 128};
static const int kBN[5] = {256, 128, 192, 64, 128};
// relative per-tile MFMA efficiency, measured on MI355X at the layer's shapes (K = 1536..3072)
static const double kEff[kNCfg] = {1.0, 0.93, 0.95};
// workgroups of each configuration resident per CU
static const int kPerCU[kNCfg] = {1, 2, 1};
static const int kCUs = 256;

// Plans measured on MI355X for the GEMMs of the 8.3B-shape layer shard (t = 8) and its
// vocabulary shard (the fastest of the three tile shapes and split counts 1..6 per shape), and for
// the weight gradients of the 1.2B attention block and the 2.5B layer where the model's pick was
// slower (layout-independent here). Other shapes use the time model below.
struct TunedPlan { int M, N, K, split_ok, cfg, splits; };
static const TunedPlan kTuned[] = {
    {8192, 1536, 3072, 0, 2, 1},   // MLP GEMM1 fwd, dU
    {8192, 3072, 1536, 0, 2, 1},   // MLP GEMM2 fwd, dX
    {8192, 1152, 3072, 0, 2, 1},   // QKV fwd
    {8192, 3072, 384, 0, 2, 1},    // output projection fwd
    {8192, 384, 3072, 0, 4, 1},    // dO (192 tiles: one three-stage workgroup per CU)
    {8192, 3072, 1152, 0, 2, 1},   // dXn
    {6400, 8192, 3072, 0, 1, 1},   // vocabulary logits (stored, and their gradient)
    {1536, 3072, 8192, 1, 0, 3},   // dB
    {3072, 1536, 8192, 1, 0, 3},   // dA
    {384, 3072, 8192, 1, 1, 6},    // dWo
    {3072, 1152, 8192, 1, 0, 4},   // dWqkv (240 units of 256x256)
    // the 1.2B attention block (t = 2) and the 2.5B layer (t = 4)
    {1536, 2304, 8192, 1, 0, 4},   // 1.2B dWqkv: 216 units of 256x256 (the model picks 432 of 128x128)
    {1920, 1920, 8192, 1, 0, 4},   // 2.5B dB, dA: 256 units of 256x256 (the model picks 450 of 128x128)
};

// Time model over the three tile shapes and split counts: rounds of resident tiles x per-tile
// MFMA time + a fixed per-round cost, plus the split-K reduction's traffic. bk = K tile depth,
// peak = dense MFMA rate of the element type; cfg_mask = tile shapes allowed (bit c).
static GemmPlan plan_model(int M, int N, int K, bool allow_split, int bk, double peak, int cfg_mask) {
    const double cu_flops = peak / kCUs * 0.8;     // sustained per-CU rate at full efficiency
    const double round_overhead = 2.0e-6;          // prologue + epilogue per wave of tiles
    GemmPlan best{1, 1, 128, 128};   // cfg 1 is always allowed
    double best_t = 1e30;
    static const int splits_opt[] = {1, 2, 3, 4, 6, 8};
    for (int c = 0; c < kNCfg; ++c) {
        if (!((cfg_mask >> c) & 1)) continue;
        for (int s : splits_opt) {
            if (s > 1 && (!allow_split || K / s < 512)) continue;
            long tiles = (long)((M + kBM[c] - 1) / kBM[c]) * ((N + kBN[c] - 1) / kBN[c]);
            long units = tiles * s;
            long slots = (long)kCUs * kPerCU[c];
            long rounds = (units + slots - 1) / slots;
            long kc = ((K + s - 1) / s + bk - 1) / bk * bk;
            double t_tile = 2.0 * kBM[c] * kBN[c] * (double)kc * kPerCU[c] / (cu_flops * kEff[c]);
            double t = rounds * (t_tile + round_overhead);
            if (s > 1) t += (s + 1.0) * 4.0 * (double)M * N / 4.0e12 + 3.0e-6;
            if (t < best_t * 0.999) { best_t = t; best = GemmPlan{c, s, kBM[c], kBN[c]}; }
        }
    }
    return best;
}

GemmPlan plan_gemm_bf16(int M, int N, int K, bool allow_split) {
    for (const TunedPlan& t : kTuned)
        if (t.M == M && t.N == N && t.K == K && (t.splits == 1 || (allow_split && t.split_ok)))
            return GemmPlan{t.cfg, t.splits, kBM[t.cfg], kBN[t.cfg]};
    return plan_model(M, N, K, allow_split, 64, 2.5e15, 7);
}

// fp8: 256x256 is left out (its fragments and accumulators exceed 256 registers per lane and
// spill).
GemmPlan plan_gemm_fp8(int M, int N, int K, bool allow_split) {
    return plan_model(M, N, K, allow_split, 128, 5.0e15, 6);
}

VocabPlan plan_vocab(int Vt, int N, int K) {
    VocabPlan v;
    const long tn = (N + 255) / 256, total = (long)((Vt + 255) / 256) * tn, rounds = total / kCUs;
    const long rows_main = tn > 0 ? rounds * kCUs / tn : 0;
    if (rounds == 0 || total % kCUs == 0 || rows_main == 0 || rows_main * 256 >= Vt) {
        v.main = (rounds > 0 && total % kCUs == 0) ? GemmPlan{0, 1, 256, 256} : plan_gemm_bf16(Vt, N, K, false);
        v.main_rows = Vt;
        v.tail = v.main;
        v.tiles_m = (Vt + v.main.bm - 1) / v.main.bm;
        return v;
    }
    v.main = GemmPlan{0, 1, 256, 256};
    v.tail = GemmPlan{3, 1, 64, 64};
    v.main_rows = (int)rows_main * 256;
    v.tiles_m = (int)rows_main + (Vt - v.main_rows + 63) / 64;
    return v;
}

RowSplitPlan plan_row_split(int M, int N, int K, bool both_kcontig) {
    RowSplitPlan v;
    v.main = plan_gemm_bf16(M, N, K, false);
    v.main_rows = M;
    v.tail = v.main;
    const long tn = (N + v.main.bn - 1) / v.main.bn, tm = (M + v.main.bm - 1) / v.main.bm;
    const long slots = (long)kCUs * (v.main.cfg == 1 ? 2 : 1);
    const long rounds = tm * tn / slots;
    if (v.main.splits != 1 || rounds == 0 || (tm * tn) % slots == 0 || (rounds * slots) % tn != 0) return v;
    const long rows_main = rounds * slots / tn * v.main.bm;
    if (rows_main >= M) return v;
    // the remaining rows on small tiles: one round of them at two workgroups per CU
    const GemmPlan tail = both_kcontig ? GemmPlan{3, 1, 64, 64} : GemmPlan{1, 1, 128, 128};
    const long tail_tiles = ((M - rows_main + tail.bm - 1) / tail.bm) * ((N + tail.bn - 1) / tail.bn);
    if (tail_tiles > 2L * kCUs) return v;
    v.main_rows = (int)rows_main;
    v.tail = tail;
    return v;
}

size_t split_ws_bytes(const GemmPlan& p, int M, int N) {
    return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_bf16(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    if (r.M == 0 || r.N == 0) return hipSuccess;
    if (!r.a_mn && r.b_mn) return gemm_bf16_nn(r, p, ws, st);
    if (!r.a_mn && !r.b_mn) return gemm_bf16_nt(r, p, ws, st);
    if (r.a_mn && r.b_mn) return gemm_bf16_tn(r, p, ws, st);
    return hipErrorInvalidValue;
}

}  // namespace tp
