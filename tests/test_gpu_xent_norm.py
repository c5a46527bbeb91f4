"""GPU parity of the vocabulary-parallel fused logits + cross-entropy statistics, the rank merge,
LayerNorm forward/backward, the partial sum and the column sums, through the C ABI.

Float tolerances: relative L2 <= 1e-2 for bf16 inputs (fp32 accumulation), <= 1e-5 for fp32.
Max and argmax are bit-exact against the GPU's own fp32 logits (same kernel, materialised)."""
import numpy as np
import pytest
import torch

import oracle
import tp_synth
from tests.gpu_util import dev, dev_i32, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")


def run_xent(inp, N, h, Vpad, Vreal, t, ranks, mask):
    X = dev(inp["X"], "bf16")
    tg = dev_i32(inp["targets"])
    Vt = Vpad // t
    out = {}
    for r in ranks:
        E_r = dev(inp["E"][r * Vt:(r + 1) * Vt], "bf16")
        mx, se, tv = empty((N,), "f32"), empty((N,), "f32"), empty((N,), "f32")
        am = torch.empty((N,), dtype=torch.int32, device="cuda:0")
        nb = tp.tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, tp.TP_BF16)
        tp.tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, r, tp.TP_BF16, mask, X, E_r, tg, mx, se, tv, am, ws(nb), nb)
        logits = empty((N, Vt), "f32")
        tp.tp_vocab_logits_shard(N, h, Vpad, t, r, tp.TP_BF16, X, E_r, logits)
        out[r] = dict(max=mx, sumexp=se, tgt=tv, argmax=am, logits=logits)
    return out


def check_bitexact_from_logits(o, r, Vt, Vreal, mask, targets):
    """max / argmax / target pick-out against the kernel's own fp32 logits, bit for bit."""
    L = o["logits"].cpu().numpy().astype(np.float32)
    if mask:
        cols = r * Vt + np.arange(Vt)
        L = np.where(cols[None, :] < Vreal, L, -np.inf).astype(np.float32)
    mx = o["max"].cpu().numpy()
    am = o["argmax"].cpu().numpy()
    assert np.array_equal(mx, L.max(axis=1))
    assert np.array_equal(am, L.argmax(axis=1) + r * Vt)
    local = targets.astype(np.int64) - r * Vt
    own = (local >= 0) & (local < Vt)
    n = np.arange(L.shape[0])
    want_t = np.where(own, L[n, np.clip(local, 0, Vt - 1)], 0.0).astype(np.float32)
    assert np.array_equal(o["tgt"].cpu().numpy(), want_t)


def check_stats_pass(o, N, Vpad, Vreal, t, r, mask, tg):
    """The statistics pass over the stored logits against the fused call's outputs: max, argmax and
    target logit bit for bit; the sum of exponentials (a different summation order) to 1e-5
    element-wise relative (fp32 sums of up to V_t terms in either order)."""
    Vt = Vpad // t
    mx, se, tv = empty((N,), "f32"), empty((N,), "f32"), empty((N,), "f32")
    am = torch.full((N,), -7, dtype=torch.int32, device="cuda:0")
    tp.tp_vocab_xent_stats_from_logits(N, Vpad, Vreal, t, r, mask, o["logits"], Vt, tg, mx, se, tv, am)
    torch.cuda.synchronize()
    assert torch.equal(mx, o["max"]) and torch.equal(am, o["argmax"]) and torch.equal(tv, o["tgt"]), r
    a, b = host(se), host(o["sumexp"])
    fin = b > 0
    assert np.array_equal(a[~fin], b[~fin])
    rel = np.abs(a[fin] - b[fin]) / b[fin]
    assert rel.size == 0 or rel.max() <= 1e-5, (r, rel.max())
    return float(rel.max()) if rel.size else 0.0


@pytest.mark.parametrize("Vreal,t,r,mask", [(1000, 4, 1, 0), (1000, 4, 3, 1), (560, 4, 3, 1), (1021, 1, 0, 1)])
def test_xent_stats_pass_small(Vreal, t, r, mask):
    """The statistics pass over materialised logits on ragged shapes (N = 300 tokens, h = 200,
    V_t = 256, 192 or 1024), with and without the padding mask; (560, t=4, r=3, mask) is a rank whose
    every column is padding: max -inf, sum 0, argmax -1, target 0."""
    N, h = 300, 200
    Vpad = oracle.pad_vocab(Vreal, t, multiple=64 if t > 1 else 1024)
    inp = tp_synth.xent_inputs(90 + Vreal + r, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    say(f"[xent] stats pass N={N} Vpad={Vpad} Vreal={Vreal} t={t} r={r} mask={mask}")
    o = run_xent(inp, N, h, Vpad, Vreal, t, [r], mask)[r]
    rel = check_stats_pass(o, N, Vpad, Vreal, t, r, mask, dev_i32(inp["targets"]))
    st = oracle.xent_shard_stats(inp["X"], oracle.vocab_shard(inp["E"], t, r), inp["targets"], t, r, Vreal, bool(mask))
    if mask and r * (Vpad // t) >= Vreal:
        assert np.all(host(o["max"]) == -np.inf) and np.all(host(o["argmax"]) == -1)
        assert np.all(host(o["sumexp"]) == 0) and np.all(host(o["tgt"]) == 0)
    else:
        for k in ("max", "sumexp", "tgt"):
            assert within(rel_l2(host(o[k]), st[k]), 1e-2), k
    say(f"[xent] stats pass: max/argmax/target equal to the fused call; sumexp max rel diff {rel:.1e}")


@pytest.mark.parametrize("mask", [0, 1])
def test_xent_small_ragged(mask):
    """N=300 tokens, h=200, Vreal=1000 padded to 1024 for t=4 (V_t=256), all ranks + merge."""
    N, h, Vreal, t = 300, 200, 1000, 4
    Vpad = oracle.pad_vocab(Vreal, t, multiple=64)
    inp = tp_synth.xent_inputs(95, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    say(f"[xent] small N={N} h={h} Vpad={Vpad} Vreal={Vreal} t={t} mask={mask}")
    out = run_xent(inp, N, h, Vpad, Vreal, t, range(t), mask)
    st = [oracle.xent_shard_stats(inp["X"], oracle.vocab_shard(inp["E"], t, r), inp["targets"], t, r, Vreal, bool(mask))
          for r in range(t)]
    Vt = Vpad // t
    for r in range(t):
        check_bitexact_from_logits(out[r], r, Vt, Vreal, mask, inp["targets"])
        for k in ("max", "sumexp", "tgt"):
            e = rel_l2(host(out[r][k]), st[r][k])
            assert within(e, 1e-2), (r, k, e)
    loss, mean = empty((N,), "f32"), empty((1,), "f32")
    tp.tp_vocab_xent_combine(N, t, [out[r]["max"] for r in range(t)], [out[r]["sumexp"] for r in range(t)],
                             [out[r]["tgt"] for r in range(t)], loss, mean)
    ref = oracle.xent_full(inp["X"], inp["E"], inp["targets"], Vreal, bool(mask))["loss"]
    e = rel_l2(host(loss), ref)
    say(f"[xent] small mask={mask}: loss rel-L2 {e:.2e}, mean {host(mean)[0]:.6f} vs {ref.mean():.6f}")
    assert within(e, 1e-2)
    assert abs(host(mean)[0] - ref.mean()) <= 1e-2 * abs(ref.mean())


@pytest.mark.parametrize("mask,h", [(1, 136), (0, 520)])
def test_xent_two_part_launch(mask, h):
    """A shard whose 256x256 tiles overflow whole rounds over the 256 CUs (V_t = 4160 rows,
    N = 4136 tokens: 17 x 17 tiles): the library runs 256x256 tiles over the first 3840 rows and
    64x64 tiles (four LDS stages) over the last 320, which hold the padded rows of the last rank
    (Vreal = 8300 of Vpad = 8320, t = 2). h = 136 gives fewer K tiles than stages, h = 520 two
    rounds of stages and one more tile. Both ranks against the oracle; max, argmax and target
    logits bit-exact against the kernel's own fp32 logits."""
    N, Vreal, t, Vpad = 4136, 8300, 2, 8320
    inp = tp_synth.xent_inputs(97 + h, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    say(f"[xent] two-part launch N={N} h={h} Vpad={Vpad} mask={mask}")
    out = run_xent(inp, N, h, Vpad, Vreal, t, range(t), mask)
    Vt = Vpad // t
    for r in range(t):
        check_bitexact_from_logits(out[r], r, Vt, Vreal, mask, inp["targets"])
        st = oracle.xent_shard_stats(inp["X"], oracle.vocab_shard(inp["E"], t, r), inp["targets"], t, r, Vreal,
                                     bool(mask))
        for k in ("max", "sumexp", "tgt"):
            e = rel_l2(host(out[r][k]), st[k])
            assert within(e, 1e-2), (r, k, e)
    # the argmax lands in the 64x64 part for some tokens
    am = out[0]["argmax"].cpu().numpy()
    assert (am >= 3840).any() and (am < 3840).any()


def argmax_vs_fp64(am_gpu, y, col0):
    """Argmax against the float64 logits y [N, V] of the same columns: equal wherever the float64
    top-2 gap of the token exceeds 1e-4 max |y| of its row (the float32 logits differ from the
    float64 ones by ~1e-6 here, so a smaller gap is a near-tie either side may break). Returns
    the number of excluded near-ties. Their expected share: the gap between the two largest of
    V_t ~ N(0, 1.1^2) logits (V_t = 6400) is ~0.3 on average and roughly uniform near 0, so a gap
    below 1e-4 * max|y| ~ 5e-4 occurs for ~0.2 % of the tokens; the tests allow 1 %."""
    top2 = np.partition(y, -2, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    clear = gap > 1e-4 * np.abs(y).max(axis=1)
    want = y.argmax(axis=1) + col0
    bad = np.flatnonzero(clear & (am_gpu != want))
    assert bad.size == 0, f"argmax differs from float64 on {bad.size} tokens, first {bad[:8]}"
    return int((~clear).sum())


@pytest.fixture(scope="module")
def xent_8p3b():
    """The 8.3B vocabulary workload on the device: N = 8192 tokens, h = 3072, Vpad = 51,200
    (t = 8, V_t = 6400), Vreal = 50,257; every rank's fused statistics, and its materialised fp32
    logits for the bit-exact checks."""
    w = tp_synth.WORKLOADS["xent_8p3b_t8"]
    inp = tp_synth.xent_inputs(w.seed, w.T, w.h, w.vocab, w.vocab_pad, "bf16")
    say("[xent] 8.3B workload: all 8 ranks on the device")
    out = run_xent(inp, w.T, w.h, w.vocab_pad, w.vocab, w.t, range(w.t), 0)
    host_out = {}
    tg = dev_i32(inp["targets"])
    for r in range(w.t):
        o = out[r]
        host_out[r] = {k: o[k].cpu().numpy() for k in ("max", "sumexp", "tgt", "argmax")}
        check_bitexact_from_logits(o, r, w.vocab_pad // w.t, w.vocab, 0, inp["targets"])
        check_stats_pass(o, w.T, w.vocab_pad, w.vocab, w.t, r, 0, tg)
    loss = empty((w.T,), "f32")
    mean = empty((1,), "f32")
    tp.tp_vocab_xent_combine(w.T, w.t, [out[r]["max"] for r in range(w.t)], [out[r]["sumexp"] for r in range(w.t)],
                             [out[r]["tgt"] for r in range(w.t)], loss, mean)
    del out
    torch.cuda.empty_cache()
    return w, inp, host_out, host(loss), float(host(mean)[0])


def test_xent_8p3b_every_rank_full_size(xent_8p3b):
    """Every rank's per-token max, sum of exponentials and target logit over all 8192 tokens
    against the float64 oracle element by element; every argmax equal to the float64 argmax
    wherever the float64 top-2 gap is clear (near-ties counted and reported)."""
    w, inp, got, _, _ = xent_8p3b
    Vt = w.vocab_pad // w.t
    ties = 0
    for r in range(w.t):
        E_r = oracle.vocab_shard(inp["E"], w.t, r)
        st = oracle.xent_shard_stats(inp["X"], E_r, inp["targets"], w.t, r, w.vocab)
        errs = {k: rel_l2(got[r][k], st[k]) for k in ("max", "sumexp", "tgt")}
        n = argmax_vs_fp64(got[r]["argmax"], st["logits"], r * Vt)
        ties += n
        say(f"[xent] 8.3B rank {r}: " + " ".join(f"{k}={v!r}" for k, v in errs.items()) + f"; argmax near-ties {n}")
        for k, e in errs.items():
            assert within(e, 1e-2), (r, k, e)
    say(f"[xent] 8.3B: argmax equal to float64 on every clear token; {ties} near-ties of {w.t * w.T} excluded")
    assert ties <= w.t * w.T // 100


def test_xent_8p3b_loss_full_size(xent_8p3b):
    """The merged loss of all 8192 tokens and its mean against full-vocabulary cross-entropy in
    float64 (the unsplit definition, over the whole padded vocabulary), in chunks of 1024 tokens;
    the global argmax (the rank whose max is largest, its argmax) against the float64 argmax."""
    w, inp, got, loss, mean = xent_8p3b
    ref, amax = [], []
    Vt = w.vocab_pad // w.t
    for c in range(0, w.T, 1024):
        f = oracle.xent_full(inp["X"][c:c + 1024], inp["E"], inp["targets"][c:c + 1024], w.vocab)
        ref.append(f["loss"])
        mx = np.stack([got[r]["max"][c:c + 1024] for r in range(w.t)])
        best = mx.argmax(axis=0)     # lowest rank on equal maxima: the lowest global column
        am = np.stack([got[r]["argmax"][c:c + 1024] for r in range(w.t)])[best, np.arange(best.size)]
        amax.append(argmax_vs_fp64(am, f["logits"], 0))
    ref = np.concatenate(ref)
    e = rel_l2(loss, ref)
    say(f"[xent] 8.3B loss {e!r}; mean {mean:.6f} vs {ref.mean():.6f}; global argmax near-ties {sum(amax)}")
    assert within(e, 1e-2)
    assert abs(mean - ref.mean()) <= 1e-2 * abs(ref.mean())
    assert sum(amax) <= w.T // 100


@pytest.mark.parametrize("dtype,h", [("f32", 136), ("bf16", 3072), ("bf16", 1920), ("f32", 4096)])
def test_layernorm_fwd_bwd(dtype, h):
    T = 333
    g = np.random.default_rng(96)
    x = tp_synth.round_to_dtype(g.standard_normal((T, h)) * 2 + 0.5, dtype)
    gam = tp_synth.round_to_dtype(1 + 0.1 * g.standard_normal(h), dtype)
    bet = tp_synth.round_to_dtype(0.1 * g.standard_normal(h), dtype)
    dy = tp_synth.round_to_dtype(g.standard_normal((T, h)), dtype)
    dres = tp_synth.round_to_dtype(g.standard_normal((T, h)), dtype)
    dt = tp.TP_BF16 if dtype == "bf16" else tp.TP_F32
    xd, gd, bd = dev(x, dtype), dev(gam, dtype), dev(bet, dtype)
    y, mean, rstd = empty((T, h), dtype), empty((T,), "f32"), empty((T,), "f32")
    tp.tp_layernorm_fwd(T, h, dt, 1e-5, xd, gd, bd, y, mean, rstd)
    dx, dg, db = empty((T, h), dtype), empty((h,), dtype), empty((h,), dtype)
    sr, sx = empty((h,), dtype), empty((h,), dtype)
    nb = tp.tp_layernorm_bwd_workspace(T, h, dt)
    tp.tp_layernorm_bwd(T, h, dt, xd, gd, mean, rstd, dev(dy, dtype), dev(dres, dtype), dx, dg, db, sr, sx, 0,
                        ws(nb), nb)
    f = oracle.layernorm_fwd(x, gam, bet)
    b = oracle.layernorm_bwd(x, gam, f["mean"], f["rstd"], dy)
    tol = 1e-5 if dtype == "f32" else 1e-2
    dx_ref = b["dx"] + dres
    errs = {"y": rel_l2(host(y), f["y"]), "mean": rel_l2(host(mean), f["mean"]), "rstd": rel_l2(host(rstd), f["rstd"]),
            "dx": rel_l2(host(dx), dx_ref), "dgamma": rel_l2(host(dg), b["dgamma"]),
            "dbeta": rel_l2(host(db), b["dbeta"]), "colsum_dres": rel_l2(host(sr), dres.sum(axis=0)),
            "colsum_dx": rel_l2(host(sx), dx_ref.sum(axis=0))}
    say(f"[ln] {dtype} h={h}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, tol), (k, e)


def test_sum_partials_and_colsum_exact():
    """Sum of small integers is exact in fp32: the device sum must equal the integer sum."""
    g = np.random.default_rng(97)
    rows, cols, t = 77, 264, 5
    parts = [g.integers(-8, 8, (rows, cols)).astype(np.float64) for _ in range(t)]
    bias = g.integers(-4, 4, cols).astype(np.float64)
    res = g.integers(-4, 4, (rows, cols)).astype(np.float64)
    out = empty((rows, cols), "f32")
    tp.tp_sum_partials(rows, cols, t, tp.TP_BF16, [dev(p, "bf16") for p in parts], dev(bias, "f32"), dev(res, "f32"),
                       out, tp.TP_F32)
    assert np.array_equal(host(out), sum(parts) + bias + res)
    cs = empty((cols,), "f32")
    nb = tp.tp_colsum_workspace(rows, cols, tp.TP_F32)
    tp.tp_colsum(rows, cols, tp.TP_F32, dev(parts[0], "f32"), cs, 0, ws(nb), nb)
    assert np.array_equal(host(cs), parts[0].sum(axis=0))


def test_layernorm_bwd_colsums_exact_and_zero_rows():
    """The fused column sum of dres is an exact integer sum for small-integer dres; with no rows
    every requested column sum is written as zero (accumulate=0) or left unchanged (accumulate=1)."""
    g = np.random.default_rng(98)
    T, h = 203, 264
    x = tp_synth.round_to_dtype(g.standard_normal((T, h)), "f32")
    gam = tp_synth.round_to_dtype(1 + 0.1 * g.standard_normal(h), "f32")
    dy = tp_synth.round_to_dtype(g.standard_normal((T, h)), "f32")
    dres = g.integers(-8, 8, (T, h)).astype(np.float64)
    f = oracle.layernorm_fwd(x, gam, np.zeros(h))
    xd, gd = dev(x, "f32"), dev(gam, "f32")
    mean, rstd = dev(f["mean"], "f32"), dev(f["rstd"], "f32")
    dx, sr = empty((T, h), "f32"), empty((h,), "f32")
    nb = tp.tp_layernorm_bwd_workspace(T, h, tp.TP_F32)
    tp.tp_layernorm_bwd(T, h, tp.TP_F32, xd, gd, mean, rstd, dev(dy, "f32"), dev(dres, "f32"), dx, None, None, sr,
                        None, 0, ws(nb), nb)
    assert np.array_equal(host(sr), dres.sum(axis=0))
    outs = [torch.full((h,), 3.0, dtype=torch.float32, device="cuda:0") for _ in range(4)]
    for acc, want in ((1, 3.0), (0, 0.0)):
        tp.tp_layernorm_bwd(0, h, tp.TP_F32, xd, gd, mean, rstd, dev(dy, "f32"), dev(dres, "f32"), dx, *outs, acc,
                            None, 0)
        for o in outs:
            assert np.array_equal(host(o), np.full(h, want))


@pytest.mark.parametrize("dtype,h,t", [("bf16", 3072, 1), ("bf16", 1920, 3), ("f32", 136, 2)])
def test_sum_partials_layernorm(dtype, h, t):
    """out = sum of partials + bias + residual (exact on small integers), then LayerNorm of the
    stored out against the oracle."""
    T = 203
    g = np.random.default_rng(99)
    parts = [g.integers(-8, 8, (T, h)).astype(np.float64) for _ in range(t)]
    bias = g.integers(-4, 4, h).astype(np.float64)
    res = g.integers(-4, 4, (T, h)).astype(np.float64)
    gam = tp_synth.round_to_dtype(1 + 0.1 * g.standard_normal(h), dtype)
    bet = tp_synth.round_to_dtype(0.1 * g.standard_normal(h), dtype)
    dt = tp.TP_BF16 if dtype == "bf16" else tp.TP_F32
    out, y = empty((T, h), dtype), empty((T, h), dtype)
    mean, rstd = empty((T,), "f32"), empty((T,), "f32")
    tp.tp_sum_partials_layernorm(T, h, t, dt, [dev(p, dtype) for p in parts], dev(bias, dtype), dev(res, dtype), out,
                                 1e-5, dev(gam, dtype), dev(bet, dtype), y, mean, rstd)
    x = sum(parts) + bias + res
    assert np.array_equal(host(out), x)
    f = oracle.layernorm_fwd(x, gam, bet)
    tol = 1e-5 if dtype == "f32" else 1e-2
    errs = {"y": rel_l2(host(y), f["y"]), "mean": rel_l2(host(mean), f["mean"]), "rstd": rel_l2(host(rstd), f["rstd"])}
    say(f"[addln] {dtype} h={h} t={t}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, tol), (k, e)
