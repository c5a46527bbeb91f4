"""Pins of the oracle's LayerNorm, pre-LN layer and vocabulary-parallel cross-entropy.
Nothing here runs on a GPU."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import tp_synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def test_layernorm_against_torch():
    g = np.random.default_rng(20)
    x = g.standard_normal((9, 40)) * 3 + 1
    gam = 1 + 0.2 * g.standard_normal(40)
    bet = 0.2 * g.standard_normal(40)
    dy = g.standard_normal((9, 40))
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    gt = torch.from_numpy(gam.copy()).requires_grad_(True)
    bt = torch.from_numpy(bet.copy()).requires_grad_(True)
    y = torch.nn.functional.layer_norm(xt, (40,), gt, bt, eps=1e-5)
    (y * torch.from_numpy(dy)).sum().backward()
    f = oracle.layernorm_fwd(x, gam, bet)
    assert _rel(f["y"], y.detach().numpy()) < 1e-14
    b = oracle.layernorm_bwd(x, gam, f["mean"], f["rstd"], dy)
    assert _rel(b["dx"], xt.grad.numpy()) < 1e-12
    assert _rel(b["dgamma"], gt.grad.numpy()) < 1e-13
    assert _rel(b["dbeta"], bt.grad.numpy()) < 1e-14


def test_layernorm_unit_gain_invariant():
    g = np.random.default_rng(21)
    x = g.standard_normal((5, 64)) * 0.01
    f = oracle.layernorm_fwd(x, np.ones(64), np.zeros(64))
    var = x.var(axis=1)
    assert np.allclose(f["y"].mean(axis=1), 0, atol=1e-15)
    assert np.allclose(f["y"].var(axis=1), var / (var + 1e-5), rtol=1e-12)


def _layer_case(b=1, s=4, h=8, heads=2, ffn=32, seed=22):
    p = tp_synth.layer_inputs(seed, b, s, h, ffn, "f32", bias_std=0.3, ln_random=True)
    # larger weights than the workload draw so that every term matters at these tiny sizes
    for k in ("Wqkv", "Wo", "A", "B"):
        p[k] = p[k] * 15
    return p


@pytest.mark.parametrize("t", [1, 2])
def test_layer_split_equals_unsplit(t):
    p = _layer_case(b=2, s=5, h=16, heads=4, ffn=64)
    f = oracle.layer_fwd(p["x"], p, 2, 5, 4)
    fs = oracle.layer_split_fwd(p["x"], p, 2, 5, 4, t)
    assert _rel(fs["x2"], f["x2"]) < 1e-13
    g = oracle.layer_bwd(p["x"], p, f, p["G"], 2, 5, 4)
    gs = oracle.layer_split_bwd(p["x"], p, fs, p["G"], 2, 5, 4, t)
    assert _rel(gs["dx"], g["dx"]) < 1e-12
    for k in ("dln1_g", "dln1_b", "dln2_g", "dln2_b"):
        assert _rel(gs[k], g[k]) < 1e-12


def test_layer_against_torch_autograd():
    """An independent pre-LN layer built from PyTorch float64 layer_norm, SDPA and gelu."""
    b, s, h, heads, ffn = 2, 5, 16, 4, 64
    p = _layer_case(b, s, h, heads, ffn)
    T = {k: torch.from_numpy(np.asarray(v, dtype=np.float64).copy()).requires_grad_(True)
         for k, v in p.items() if k not in ("G",)}
    F = torch.nn.functional
    d = h // heads
    x = T["x"]
    xn = F.layer_norm(x, (h,), T["ln1_g"], T["ln1_b"], eps=1e-5)
    qkv = xn @ T["Wqkv"] + T["bqkv"]
    q, k, v = (qkv[:, i * h:(i + 1) * h].reshape(b, s, heads, d).transpose(1, 2) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(1, 2).reshape(b * s, h)
    x1 = x + o @ T["Wo"] + T["bo"]
    x2 = x1 + F.gelu(F.layer_norm(x1, (h,), T["ln2_g"], T["ln2_b"], eps=1e-5) @ T["A"] + T["b1"]) @ T["B"] + T["b2"]
    (x2 * torch.from_numpy(p["G"])).sum().backward()
    f = oracle.layer_split_fwd(p["x"], p, b, s, heads, 2)
    assert _rel(f["x2"], x2.detach().numpy()) < 1e-13
    g = oracle.layer_split_bwd(p["x"], p, f, p["G"], b, s, heads, 2)
    assert _rel(g["dx"], T["x"].grad.numpy()) < 1e-12
    assert _rel(g["mlp"]["dA"], T["A"].grad.numpy()) < 1e-12
    assert _rel(g["attn"]["dWqkv"], T["Wqkv"].grad.numpy()) < 1e-12
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        assert _rel(g["d" + k], T[k].grad.numpy()) < 1e-12, k


def test_layer_against_torch_transformer_encoder_layer():
    """The whole unsplit layer, forward and backward, against PyTorch's own pre-LN encoder layer
    (torch.nn.TransformerEncoderLayer with norm_first, erf GeLU, no dropout, a causal mask) in
    float64: a library composition of the block, independent of the oracle's."""
    b, s, h, heads, ffn = 2, 6, 16, 4, 64
    p = _layer_case(b, s, h, heads, ffn)
    layer = torch.nn.TransformerEncoderLayer(h, heads, dim_feedforward=ffn, dropout=0.0, activation="gelu",
                                             layer_norm_eps=1e-5, batch_first=True, norm_first=True,
                                             dtype=torch.float64)
    t64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(t64(p["Wqkv"].T))
        layer.self_attn.in_proj_bias.copy_(t64(p["bqkv"]))
        layer.self_attn.out_proj.weight.copy_(t64(p["Wo"].T))
        layer.self_attn.out_proj.bias.copy_(t64(p["bo"]))
        layer.linear1.weight.copy_(t64(p["A"].T))
        layer.linear1.bias.copy_(t64(p["b1"]))
        layer.linear2.weight.copy_(t64(p["B"].T))
        layer.linear2.bias.copy_(t64(p["b2"]))
        for norm, k in ((layer.norm1, "ln1"), (layer.norm2, "ln2")):
            norm.weight.copy_(t64(p[k + "_g"]))
            norm.bias.copy_(t64(p[k + "_b"]))
    x = t64(p["x"]).reshape(b, s, h).requires_grad_(True)
    mask = torch.nn.Transformer.generate_square_subsequent_mask(s, dtype=torch.float64)
    out = layer(x, src_mask=mask, is_causal=True)
    (out * t64(p["G"]).reshape(b, s, h)).sum().backward()
    f = oracle.layer_fwd(p["x"], p, b, s, heads)
    g = oracle.layer_bwd(p["x"], p, f, p["G"], b, s, heads)
    assert _rel(f["x2"], out.detach().reshape(b * s, h).numpy()) < 1e-13
    assert _rel(g["dx"], x.grad.reshape(b * s, h).numpy()) < 1e-12
    want = {("attn", "dWqkv"): layer.self_attn.in_proj_weight.grad.T, ("attn", "dbqkv"): layer.self_attn.in_proj_bias.grad,
            ("attn", "dWo"): layer.self_attn.out_proj.weight.grad.T, ("attn", "dbo"): layer.self_attn.out_proj.bias.grad,
            ("mlp", "dA"): layer.linear1.weight.grad.T, ("mlp", "db1"): layer.linear1.bias.grad,
            ("mlp", "dB"): layer.linear2.weight.grad.T, ("mlp", "db2"): layer.linear2.bias.grad}
    for (blk, k), ref in want.items():
        assert _rel(g[blk][k], ref.numpy()) < 1e-12, k
    for k, norm in (("ln1", layer.norm1), ("ln2", layer.norm2)):
        assert _rel(g["d" + k + "_g"], norm.weight.grad.numpy()) < 1e-12, k
        assert _rel(g["d" + k + "_b"], norm.bias.grad.numpy()) < 1e-12, k


def test_layer_finite_differences_input():
    b, s, h, heads, ffn = 1, 4, 8, 2, 32
    p = _layer_case(b, s, h, heads, ffn)
    f = oracle.layer_split_fwd(p["x"], p, b, s, heads, 2)
    g = oracle.layer_split_bwd(p["x"], p, f, p["G"], b, s, heads, 2)
    eps = 1e-6
    fd = np.zeros_like(p["x"])
    for idx in np.ndindex(p["x"].shape):
        xp, xm = p["x"].copy(), p["x"].copy()
        xp[idx] += eps
        xm[idx] -= eps
        lp = (oracle.layer_split_fwd(xp, p, b, s, heads, 2)["x2"] * p["G"]).sum()
        lm = (oracle.layer_split_fwd(xm, p, b, s, heads, 2)["x2"] * p["G"]).sum()
        fd[idx] = (lp - lm) / (2 * eps)
    assert _rel(g["dx"], fd) < 1e-7


def test_vocab_padding_geometry():
    """"Megatron-LM, annotated" §3.4: 50,257 rounds up to 51,200 (943 padding rows) for
    8 GPUs, 6,400 per GPU; logits vs losses counts."""
    g = json.load(open(os.path.join(GOLD, "geometry.json")))
    vp = oracle.pad_vocab(g["vocab"], g["gpus"])
    assert vp == g["vocab_padded"] and vp - g["vocab"] == g["padding_rows"]
    assert vp // g["gpus"] == g["vocab_per_gpu"] and (vp // g["gpus"]) % 128 == 0
    assert 8 * 1024 * vp == g["logits_per_step"] and 8 * 1024 == g["losses_per_step"]
    assert round(8 * 1024 * g["hidden_8p3b"] / 1e6, 1) == g["message_elements_millions"]
    w = tp_synth.WORKLOADS["xent_8p3b_t8"]
    assert w.vocab_pad == vp and w.per_rank()["V_t"] == g["vocab_per_gpu"]


@pytest.mark.parametrize("mask", [False, True])
@pytest.mark.parametrize("t", [1, 2, 4])
def test_xent_split_merges(mask, t):
    """One-round merge == the pages' two-round scheme == unsplit == PyTorch cross_entropy."""
    g = np.random.default_rng(23)
    N, h, Vreal = 11, 6, 29
    Vp = oracle.pad_vocab(Vreal, t, multiple=8)
    X = g.standard_normal((N, h)) * 2
    E = g.standard_normal((Vp, h))
    tg = g.integers(0, Vreal, N)
    full = oracle.xent_full(X, E, tg, Vreal, mask)
    logits = torch.from_numpy(full["logits"][:, :Vreal] if mask else full["logits"])
    ref = torch.nn.functional.cross_entropy(logits, torch.from_numpy(tg), reduction="none").numpy()
    assert _rel(full["loss"], ref) < 1e-14
    st = [oracle.xent_shard_stats(X, oracle.vocab_shard(E, t, r), tg, t, r, Vreal, mask) for r in range(t)]
    one = oracle.xent_combine([s["max"] for s in st], [s["sumexp"] for s in st], [s["tgt"] for s in st])
    two = oracle.xent_two_round(X, E, tg, t, Vreal, mask)
    assert _rel(one, ref) < 1e-14 and _rel(two, ref) < 1e-14
    # the target logit is owned by exactly one rank
    owners = np.stack([s["tgt"] != 0 for s in st]).sum(axis=0)
    assert np.all(owners == 1)
    # merged max and argmax are the full-vocabulary ones (lowest index on ties)
    mx = np.stack([s["max"] for s in st])
    am = np.stack([s["argmax"] for s in st])
    best = mx.argmax(axis=0)
    assert np.array_equal(mx.max(axis=0), full["max"])
    assert np.array_equal(am[best, np.arange(N)], full["argmax"])


def test_xent_argmax_ties_lowest_index():
    X = np.ones((1, 2))
    E = np.array([[0.0, 1.0], [1.0, 0.0], [0.25, 0.25], [1.0, 0.0]])
    st = [oracle.xent_shard_stats(X, oracle.vocab_shard(E, 2, r), np.array([0]), 2, r, 4) for r in range(2)]
    assert st[0]["argmax"][0] == 0 and st[1]["argmax"][0] == 3
    assert st[0]["max"][0] == st[1]["max"][0] == 1.0


# ---- cross-entropy backward ----------------------------------------------------------------
def _xent_case(seed, N, h, V, Vreal):
    g = np.random.default_rng(seed)
    X = g.standard_normal((N, h))
    E = 0.3 * g.standard_normal((V, h))
    tg = g.integers(0, Vreal, N)
    dl = g.uniform(0.5, 1.5, N)
    return X, E, tg, dl


@pytest.mark.parametrize("mask", [0, 1])
def test_xent_grad_against_torch_autograd(mask):
    """Unsplit gradients against PyTorch CPU float64 autograd of sum_n dloss_n * cross_entropy_n."""
    X, E, tg, dl = _xent_case(21, 9, 7, 24, 20)
    ours = oracle.xent_full_grad(X, E, tg, 20, bool(mask), dl)
    Xt = torch.tensor(X, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    y = Xt @ Et.T
    if mask:
        y = y.masked_fill(torch.arange(24)[None, :] >= 20, float("-inf"))
    loss = (torch.tensor(dl) * torch.nn.functional.cross_entropy(y, torch.tensor(tg), reduction="none")).sum()
    loss.backward()
    assert np.allclose(ours["dX"], Xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(ours["dE"], Et.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_xent_grad_finite_differences():
    """Central differences of the forward loss definition (step 1e-6) against the analytic
    gradient, on every entry of X and of E."""
    X, E, tg, dl = _xent_case(22, 4, 3, 10, 10)
    gr = oracle.xent_full_grad(X, E, tg, 10, False, dl)

    def L(Xv, Ev):
        return float((dl * oracle.xent_full(Xv, Ev, tg, 10)["loss"]).sum())

    eps = 1e-6
    for A, key in ((X, "dX"), (E, "dE")):
        num = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += eps
            Am[idx] -= eps
            args_p = (Ap, E) if key == "dX" else (X, Ap)
            args_m = (Am, E) if key == "dX" else (X, Am)
            num[idx] = (L(*args_p) - L(*args_m)) / (2 * eps)
        assert np.allclose(num, gr[key], rtol=1e-6, atol=1e-8), key


@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("t", [2, 4])
def test_xent_grad_split_sums_to_unsplit(mask, t):
    """With the merged (M, S): sum over ranks of dX_r equals the unsplit dX, the ranks' dE_r
    stack to the unsplit dE, and each token's logits gradient sums to zero over the vocabulary."""
    V, Vreal = 32, 29
    X, E, tg, dl = _xent_case(23 + t, 11, 6, V, Vreal)
    full = oracle.xent_full_grad(X, E, tg, Vreal, bool(mask), dl)
    M, S = oracle.xent_merged_stats(X, E, tg, Vreal, bool(mask))
    parts = [oracle.xent_shard_grad(X, oracle.vocab_shard(E, t, r), tg, t, r, Vreal, bool(mask), M, S, dl)
             for r in range(t)]
    assert np.allclose(sum(p["dX"] for p in parts), full["dX"], rtol=1e-12, atol=1e-13)
    assert np.allclose(np.concatenate([p["dE"] for p in parts]), full["dE"], rtol=1e-12, atol=1e-13)
    rows = np.concatenate([p["dlogits"] for p in parts], axis=1).sum(axis=1)
    assert np.allclose(rows, 0.0, atol=1e-14)
    if mask:
        assert np.all(np.concatenate([p["dlogits"] for p in parts], axis=1)[:, Vreal:] == 0.0)


def test_xent_grad_uniform_logits():
    """E = 0: every logit is 0, the softmax is uniform, dlogits = dloss * (1/V - onehot)."""
    X, _, tg, dl = _xent_case(24, 5, 4, 8, 8)
    gr = oracle.xent_full_grad(X, np.zeros((8, 4)), tg, 8, False, dl)
    want = dl[:, None] * (np.full((5, 8), 1.0 / 8) - np.eye(8)[tg])
    assert np.allclose(gr["dlogits"], want, rtol=0, atol=1e-15)
