"""Pins of the oracle's attention block: library routine, closed forms, invariants, autograd
and finite differences. Nothing here runs on a GPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


@pytest.mark.parametrize("causal", [True, False])
def test_core_matches_torch_sdpa(causal):
    g = np.random.default_rng(10)
    s, d = 37, 12
    Q, K, V = (g.standard_normal((s, d)) for _ in range(3))
    out = oracle.attn_core_fwd(Q, K, V, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None, None] for a in (Q, K, V)), is_causal=causal)[0, 0].numpy()
    assert _rel(out["O"], ref) < 1e-13
    # lse is the log of the softmax denominator: P = exp(S - lse)
    S = Q @ K.T / math.sqrt(d)
    if causal:
        S = np.where(np.tril(np.ones((s, s), bool)), S, -np.inf)
    assert np.allclose(np.exp(S - out["lse"][:, None]), out["P"], rtol=1e-13, atol=1e-15)


def test_core_special_cases():
    g = np.random.default_rng(11)
    d = 8
    V = g.standard_normal((20, d))
    # one position: the only visible key is itself, O = V
    out = oracle.attn_core_fwd(g.standard_normal((1, d)), g.standard_normal((1, d)), V[:1], True)
    assert np.array_equal(out["O"], V[:1])
    # Q = 0: all visible scores equal, causal O is the running mean of V
    out = oracle.attn_core_fwd(np.zeros((20, d)), g.standard_normal((20, d)), V, True)
    running = np.cumsum(V, axis=0) / np.arange(1, 21)[:, None]
    assert np.allclose(out["O"], running, rtol=1e-13, atol=1e-14)
    assert np.allclose(out["lse"], np.log(np.arange(1, 21)), rtol=0, atol=1e-14)


def test_core_is_causal():
    """Changing later tokens leaves earlier outputs unchanged."""
    g = np.random.default_rng(12)
    Q, K, V = (g.standard_normal((16, 8)) for _ in range(3))
    a = oracle.attn_core_fwd(Q, K, V, True)["O"]
    K2, V2 = K.copy(), V.copy()
    K2[9:] += 5.0
    V2[9:] -= 3.0
    b = oracle.attn_core_fwd(Q, K2, V2, True)["O"]
    assert np.array_equal(a[:9], b[:9])
    assert not np.allclose(a[9:], b[9:])


def _attn_case(b=2, s=6, h=16, heads=4, seed=13, bias=True):
    g = np.random.default_rng(seed)
    return dict(Xn=g.standard_normal((b * s, h)), Wqkv=g.standard_normal((h, 3 * h)) * 0.3,
                bqkv=g.standard_normal(3 * h) * (0.3 if bias else 0), Wo=g.standard_normal((h, h)) * 0.3,
                bo=g.standard_normal(h) * (0.3 if bias else 0), G=g.standard_normal((b * s, h)),
                b=b, s=s, h=h, heads=heads)


def _torch_attn(c, causal=True):
    """Independent implementation: PyTorch float64 SDPA with autograd."""
    b, s, h, heads = c["b"], c["s"], c["h"], c["heads"]
    d = h // heads
    p = {k: torch.from_numpy(c[k].copy()).requires_grad_(True) for k in ("Xn", "Wqkv", "bqkv", "Wo", "bo")}
    qkv = p["Xn"] @ p["Wqkv"] + p["bqkv"]
    q, k, v = (qkv[:, i * h:(i + 1) * h].reshape(b, s, heads, d).transpose(1, 2) for i in range(3))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    o = o.transpose(1, 2).reshape(b * s, h)
    Z = o @ p["Wo"] + p["bo"]
    (Z * torch.from_numpy(c["G"])).sum().backward()
    return Z.detach().numpy(), {k: v.grad.numpy() for k, v in p.items()}


@pytest.mark.parametrize("causal", [True, False])
def test_block_against_torch(causal):
    c = _attn_case()
    Zt, grads = _torch_attn(c, causal)
    f = oracle.attn_fwd(c["Xn"], c["Wqkv"], c["bqkv"], c["Wo"], c["bo"], c["b"], c["s"], c["heads"], causal)
    assert _rel(f["Z"], Zt) < 1e-13
    gr = oracle.attn_bwd(c["Xn"], c["Wqkv"], c["Wo"], f, c["G"], c["b"], c["s"], c["heads"])
    for k, tk in (("dXn", "Xn"), ("dWqkv", "Wqkv"), ("dbqkv", "bqkv"), ("dWo", "Wo"), ("dbo", "bo")):
        assert _rel(gr[k], grads[tk]) < 1e-12, k


@pytest.mark.parametrize("t", [1, 2, 4])
def test_head_split_equals_unsplit(t):
    """Heads are independent, so the sum of the head-sharded partials plus bo is the block
    ("Megatron-LM ..." digest §3.4, attention head parallelism); backward likewise."""
    c = _attn_case()
    f = oracle.attn_fwd(c["Xn"], c["Wqkv"], c["bqkv"], c["Wo"], c["bo"], c["b"], c["s"], c["heads"])
    sp = oracle.attn_split_fwd(c["Xn"], c["Wqkv"], c["bqkv"], c["Wo"], c["bo"], c["b"], c["s"], c["heads"], t)
    assert _rel(sp["Z"], f["Z"]) < 1e-13
    gf = oracle.attn_bwd(c["Xn"], c["Wqkv"], c["Wo"], f, c["G"], c["b"], c["s"], c["heads"])
    gs = oracle.attn_split_bwd(c["Xn"], c["Wqkv"], c["Wo"], sp["ranks"], c["G"], c["b"], c["s"], c["heads"], t)
    for k in ("dXn", "dWqkv", "dbqkv", "dWo", "dbo"):
        assert _rel(gs[k], gf[k]) < 1e-12, k
    if t > 1:
        assert _rel(gs["ranks"][0]["dXn"], gf["dXn"]) > 1e-3


def test_head_shard_geometry():
    """"Megatron-LM, annotated" §3.2: the 8.3B model's 32 heads on 8 GPUs are 4 per GPU of
    width 96; rank r's packed projection takes exactly its heads' columns of each third."""
    g = json.load(open(os.path.join(GOLD, "geometry.json")))
    h, heads, t = g["hidden_8p3b"], g["heads_8p3b"], g["gpus"]
    assert heads // t == g["heads_per_gpu"] and h // heads == g["head_width"]
    lo, hi = oracle.head_columns(h, heads, t, 3)
    assert (hi - lo) == g["heads_per_gpu"] * g["head_width"]
    W = np.arange(3 * h, dtype=np.float64)[None, :]
    Wr = oracle.qkv_shard(W, heads, t, 3)[0]
    assert Wr.shape == (3 * (hi - lo),)
    assert np.array_equal(Wr[:hi - lo], np.arange(lo, hi))
    assert np.array_equal(Wr[hi - lo:2 * (hi - lo)], h + np.arange(lo, hi))
    assert np.array_equal(Wr[2 * (hi - lo):], 2 * h + np.arange(lo, hi))


def test_attention_finite_differences():
    """b=1, s=4, 2 heads of width 4, t=2: central differences of L = sum(G * Z)."""
    c = _attn_case(b=1, s=4, h=8, heads=2, seed=14)
    t = 2

    def loss(Xn, Wqkv, bqkv, Wo, bo):
        return float((oracle.attn_split_fwd(Xn, Wqkv, bqkv, Wo, bo, 1, 4, 2, t)["Z"] * c["G"]).sum())

    sp = oracle.attn_split_fwd(c["Xn"], c["Wqkv"], c["bqkv"], c["Wo"], c["bo"], 1, 4, 2, t)
    gs = oracle.attn_split_bwd(c["Xn"], c["Wqkv"], c["Wo"], sp["ranks"], c["G"], 1, 4, 2, t)
    names = ["Xn", "Wqkv", "bqkv", "Wo", "bo"]
    args = [c[n] for n in names]
    eps = 1e-6
    for i, n in enumerate(names):
        fd = np.zeros_like(args[i])
        for idx in np.ndindex(args[i].shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[i][idx] += eps
            m[i][idx] -= eps
            fd[idx] = (loss(*p) - loss(*m)) / (2 * eps)
        assert _rel(gs["d" + n], fd) < 1e-7, n
