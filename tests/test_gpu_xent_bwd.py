"""GPU parity of the vocabulary-parallel cross-entropy backward (the gradient of the pages'
fused logits + cross-entropy, "Megatron-LM ..." digest §3.4) through the C ABI, against the
float64 oracle: rank r's dX_r (a partial whose sum over ranks is dL/dX) and dE_r.

Tolerance: relative L2 <= 1e-2 (bf16 inputs, fp32 accumulation; the logits gradient is rounded
to bf16 between the GEMMs)."""
import numpy as np
import pytest
import torch

import oracle
import tp_synth
from tests.gpu_util import dev, dev_i32, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")
TOL = 1e-2


def run_bwd(inp, N, h, Vpad, Vreal, t, r, mask, M, S, g, accumulate=0, dE0=None):
    Vt = Vpad // t
    X = dev(inp["X"], "bf16")
    E_r = dev(inp["E"][r * Vt:(r + 1) * Vt], "bf16")
    dX, dE = empty((N, h), "bf16"), (dev(dE0, "bf16") if dE0 is not None else empty((Vt, h), "bf16"))
    nb = tp.tp_vocab_xent_shard_bwd_workspace(N, h, Vpad, t, tp.TP_BF16)
    tp.tp_vocab_xent_shard_bwd(N, h, Vpad, Vreal, t, r, tp.TP_BF16, mask, X, E_r, dev_i32(inp["targets"]),
                               dev(M, "f32"), dev(S, "f32"), dev(g, "f32"), dX, dE, accumulate, ws(nb), nb)
    return host(dX), host(dE)


@pytest.mark.parametrize("mask", [0, 1])
def test_xent_bwd_small_ragged(mask):
    """N = 333 tokens (not a multiple of 8), h = 264, Vreal = 1000 padded to 1024 for t = 2;
    every rank against the oracle, and the ranks' dX partials summed against the unsplit dX."""
    N, h, Vreal, t = 333, 264, 1000, 2
    Vpad = oracle.pad_vocab(Vreal, t, multiple=64)
    inp = tp_synth.xent_inputs(501, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    g = np.random.default_rng(502).uniform(0.5, 1.5, N) / N
    M, S = oracle.xent_merged_stats(inp["X"], inp["E"], inp["targets"], Vreal, bool(mask))
    full = oracle.xent_full_grad(inp["X"], inp["E"], inp["targets"], Vreal, bool(mask), g)
    Vt = Vpad // t
    dX_sum = np.zeros((N, h))
    for r in range(t):
        dX, dE = run_bwd(inp, N, h, Vpad, Vreal, t, r, mask, M, S, g)
        ref = oracle.xent_shard_grad(inp["X"], inp["E"][r * Vt:(r + 1) * Vt], inp["targets"], t, r, Vreal,
                                     bool(mask), M, S, g)
        e = {"dX_r": rel_l2(dX, ref["dX"]), "dE_r": rel_l2(dE, ref["dE"])}
        say(f"[xent-bwd] small mask={mask} rank {r}: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
        for k, v in e.items():
            assert within(v, TOL), (r, k, v)
        if mask:
            pad = np.arange(Vt) + r * Vt >= Vreal
            assert np.all(dE[pad] == 0.0)
        dX_sum += dX
    e = rel_l2(dX_sum, full["dX"])
    say(f"[xent-bwd] small mask={mask}: sum of dX_r vs unsplit dX rel-L2 {e:.2e}")
    assert within(e, TOL)


def test_xent_bwd_row_split_ragged():
    """A shard large enough that both row splits of the backward engage, with ragged remainders:
    N = 4096 tokens, h = 3072, Vreal = 10990 padded to 10992 for t = 2 (V_t = 5496), rank 1 (which
    holds the padding rows) with the padding mask. The logits gradient runs 256x256 tiles over
    vocabulary rows 0-4095 and 64x64 tiles over the last 1400 (56 rows in the last tile row); dE_r
    runs one round of 256x192 tiles over rows 0-4095 and 128x128 tiles over the last 1400 (120 in
    the last tile row). Every element of dX_r and dE_r against the oracle."""
    N, h, Vreal, t, r = 4096, 3072, 10990, 2, 1
    Vpad = oracle.pad_vocab(Vreal, t, multiple=8)
    assert Vpad == 10992
    Vt = Vpad // t
    inp = tp_synth.xent_inputs(507, N, h, Vreal, Vpad, "bf16")
    g = np.random.default_rng(508).uniform(0.5, 1.5, N) / N
    M, S = oracle.xent_merged_stats(inp["X"], inp["E"], inp["targets"], Vreal, True)
    dX, dE = run_bwd(inp, N, h, Vpad, Vreal, t, r, 1, M, S, g)
    ref = oracle.xent_shard_grad(inp["X"], inp["E"][r * Vt:(r + 1) * Vt], inp["targets"], t, r, Vreal, True, M,
                                 S, g)
    e = {"dX_r": rel_l2(dX, ref["dX"]), "dE_r rows 0-4095": rel_l2(dE[:4096], ref["dE"][:4096]),
         "dE_r rows 4096-5495": rel_l2(dE[4096:], ref["dE"][4096:])}
    say("[xent-bwd] row split: " + " ".join(f"{k}={v!r}" for k, v in e.items()))
    for k, v in e.items():
        assert within(v, TOL), (k, v)
    pad = np.arange(Vt) + r * Vt >= Vreal
    assert pad.sum() == 2 and np.all(dE[pad] == 0.0)


def test_xent_bwd_chain_from_forward():
    """The whole chain on the device: per-rank statistics (forward), the merge with its M and S,
    then the backward; against the oracle computed from the inputs alone."""
    N, h, Vreal, t = 256, 200, 500, 2
    Vpad = oracle.pad_vocab(Vreal, t, multiple=64)
    inp = tp_synth.xent_inputs(503, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    Vt = Vpad // t
    X, tg = dev(inp["X"], "bf16"), dev_i32(inp["targets"])
    stats = []
    for r in range(t):
        mx, se, tv = empty((N,), "f32"), empty((N,), "f32"), empty((N,), "f32")
        nb = tp.tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, tp.TP_BF16)
        tp.tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, r, tp.TP_BF16, 0, X, dev(inp["E"][r * Vt:(r + 1) * Vt], "bf16"),
                                   tg, mx, se, tv, None, ws(nb), nb)
        stats.append((mx, se, tv))
    loss, M, S = empty((N,), "f32"), empty((N,), "f32"), empty((N,), "f32")
    tp.tp_vocab_xent_combine(N, t, [s[0] for s in stats], [s[1] for s in stats], [s[2] for s in stats], loss, None, M, S)
    g = torch.full((N,), 1.0 / N, dtype=torch.float32, device="cuda:0")
    dX_sum = np.zeros((N, h))
    dEs = []
    for r in range(t):
        dX, dE = empty((N, h), "bf16"), empty((Vt, h), "bf16")
        nb = tp.tp_vocab_xent_shard_bwd_workspace(N, h, Vpad, t, tp.TP_BF16)
        tp.tp_vocab_xent_shard_bwd(N, h, Vpad, Vreal, t, r, tp.TP_BF16, 0, X, dev(inp["E"][r * Vt:(r + 1) * Vt], "bf16"),
                                   tg, M, S, g, dX, dE, 0, ws(nb), nb)
        dX_sum += host(dX)
        dEs.append(host(dE))
    full = oracle.xent_full_grad(inp["X"], inp["E"], inp["targets"], Vreal, False)
    e = {"dX": rel_l2(dX_sum, full["dX"]), "dE": rel_l2(np.concatenate(dEs), full["dE"])}
    say("[xent-bwd] chain: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
    for k, v in e.items():
        assert within(v, TOL), (k, v)


def test_xent_bwd_accumulate_and_zero_tokens():
    """accumulate = 1 adds into dE_r; N = 0 writes zeros (accumulate = 0) or leaves dE_r unchanged."""
    N, h, Vreal, t, r = 64, 136, 256, 2, 1
    Vpad = 256
    inp = tp_synth.xent_inputs(504, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    g = np.full(N, 1.0 / N)
    M, S = oracle.xent_merged_stats(inp["X"], inp["E"], inp["targets"], Vreal)
    Vt = Vpad // t
    base = tp_synth.round_to_dtype(np.random.default_rng(505).standard_normal((Vt, h)) * 1e-3, "bf16")
    _, dE = run_bwd(inp, N, h, Vpad, Vreal, t, r, 0, M, S, g, accumulate=1, dE0=base)
    ref = oracle.xent_shard_grad(inp["X"], inp["E"][r * Vt:], inp["targets"], t, r, Vreal, False, M, S, g)["dE"] + base
    assert within(rel_l2(dE, ref), TOL)
    X = dev(inp["X"], "bf16")
    E_r = dev(inp["E"][r * Vt:], "bf16")
    tg = dev_i32(inp["targets"])
    for acc, want in ((1, base), (0, np.zeros_like(base))):
        dE0 = dev(base, "bf16")
        tp.tp_vocab_xent_shard_bwd(0, h, Vpad, Vreal, t, r, tp.TP_BF16, 0, X, E_r, tg, dev(M, "f32"), dev(S, "f32"),
                                   dev(g, "f32"), empty((1, h), "bf16"), dE0, acc, None, 0)
        assert np.array_equal(host(dE0), want)


def test_xent_bwd_8p3b_shard_sampled():
    """Rank 0 of the 8.3B vocabulary shard at full size (N = 8192, h = 3072, V_t = 6400). The
    merged statistics are inputs of the backward, so any positive S is a valid case: M = 8 and
    S = 51200 exp(-8) stand in for every token. dX_r is checked on 64 sampled tokens, dE_r on 96
    sampled columns (all tokens)."""
    w = tp_synth.WORKLOADS["xent_8p3b_t8"]
    N, h, t, r = w.T, w.h, w.t, 0
    Vt = w.vocab_pad // t
    inp = tp_synth.xent_inputs(w.seed, N, h, w.vocab, w.vocab_pad, "bf16")
    M = np.full(N, 8.0)
    S = np.full(N, w.vocab_pad * np.exp(-8.0))
    g = np.full(N, 1.0 / N)
    say("[xent-bwd] 8.3B shard, rank 0")
    dX, dE = run_bwd(inp, N, h, w.vocab_pad, w.vocab, t, r, 0, M, S, g)
    E_r = inp["E"][:Vt]
    rs = np.random.default_rng([w.seed, 99])
    rows = np.sort(rs.choice(N, 64, replace=False))
    cols = np.sort(rs.choice(h, 96, replace=False))
    sub = oracle.xent_shard_grad(inp["X"][rows], E_r, inp["targets"][rows], t, r, w.vocab, False, M[rows], S[rows],
                                 g[rows])
    dl = oracle.xent_shard_grad(inp["X"], E_r, inp["targets"], t, r, w.vocab, False, M, S, g)["dlogits"]
    e = {"dX_r rows": rel_l2(dX[rows], sub["dX"]), "dE_r cols": rel_l2(dE[:, cols], dl.T @ inp["X"][:, cols])}
    say("[xent-bwd] 8.3B: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()))
    for k, v in e.items():
        assert within(v, TOL), (k, v)
