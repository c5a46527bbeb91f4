"""Pins for dropout in the oracle's attention core and split layer (oracle/attention.py,
oracle/layer.py with oracle/rng.py masks): PyTorch CPU float64 autograd with the same constant
masks, the all-keep reduction, the rowsum identity the GPU backward relies on, and central
finite differences through a whole split layer with every dropout site active."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.rng as rng
import tp_synth
from tests.test_oracle_layer_xent import _layer_case, _rel

DROP = {"p": 0.3, "seed": 2024, "resid_streams": (0, 1), "attn_streams": [1000, 1001]}


def test_attention_core_dropout_against_autograd():
    g = np.random.default_rng(31)
    s, d = 40, 16
    Q, K, V, dO = (g.standard_normal((s, d)) for _ in range(4))
    keep = rng.attn_keep(0, 1, s, 2, 0.3, seed=9, stream=4)
    scale = rng.drop_scale(0.3)
    f = oracle.attn_core_fwd(Q, K, V, True, keep, scale)
    b = oracle.attn_core_bwd(Q, K, V, f["P"], dO, keep, scale)
    T = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (Q, K, V)]
    S = T[0] @ T[1].T / math.sqrt(d)
    S = S.masked_fill(~torch.tril(torch.ones(s, s, dtype=torch.bool)), float("-inf"))
    P = torch.softmax(S, dim=1)
    O = (P * torch.from_numpy(keep.astype(np.float64)) * scale) @ T[2]
    (O * torch.from_numpy(dO)).sum().backward()
    assert _rel(f["O"], O.detach().numpy()) < 1e-14
    for k, tt in zip(("dQ", "dK", "dV"), T):
        assert _rel(b[k], tt.grad.numpy()) < 1e-13, k
    # the rowsum identity: sum_k P dP = rowsum(dO * O) with the dropped O
    dP = np.where(keep, (dO @ V.T) * scale, 0.0)
    assert np.allclose((f["P"] * dP).sum(axis=1), (dO * f["O"]).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_attention_dropout_all_keep_is_plain_attention():
    g = np.random.default_rng(32)
    Q, K, V, dO = (g.standard_normal((24, 8)) for _ in range(4))
    ones = np.ones((24, 24), dtype=bool)
    a = oracle.attn_core_fwd(Q, K, V, True, ones, 1.0)
    b = oracle.attn_core_fwd(Q, K, V, True)
    assert np.array_equal(a["O"], b["O"])
    ga = oracle.attn_core_bwd(Q, K, V, a["P"], dO, ones, 1.0)
    gb = oracle.attn_core_bwd(Q, K, V, b["P"], dO)
    for k in ga:
        assert np.array_equal(ga[k], gb[k])


def test_layer_dropout_masks_and_sites():
    b, s, h, heads, ffn = 2, 6, 16, 4, 64
    p = _layer_case(b, s, h, heads, ffn)
    f = oracle.layer_split_fwd(p["x"], p, b, s, heads, 2, drop=DROP)
    k1 = rng.residual_keep(b * s, h, 0.3, 2024, 0)
    assert np.array_equal(f["keep1"], k1)
    # x1 = x + D1(attention sum + bo)
    z = sum(r["Z"] for r in f["attn"]["ranks"]) + p["bo"]
    assert _rel(f["x1"], p["x"] + rng.dropout_apply(z, k1, 0.3)) < 1e-15
    # rank r's heads use rank r's stream; the masks differ between ranks
    r0, r1 = f["attn"]["ranks"]
    assert np.array_equal(r0["keep"][1, 0], rng.attn_keep(1, 0, s, heads, 0.3, 2024, 1000))
    assert np.array_equal(r1["keep"][0, 1], rng.attn_keep(0, 3, s, heads, 0.3, 2024, 1001))
    assert not np.array_equal(r0["keep"][0, 0], rng.attn_keep(0, 0, s, heads, 0.3, 2024, 1001))


def test_layer_dropout_finite_differences():
    b, s, h, heads, ffn = 1, 4, 8, 2, 32
    p = _layer_case(b, s, h, heads, ffn)
    f = oracle.layer_split_fwd(p["x"], p, b, s, heads, 2, drop=DROP)
    # every site drops something at these sizes
    assert not f["keep1"].all() and not f["keep2"].all()
    assert not all(k.all() for r in f["attn"]["ranks"] for k in r["keep"].values())
    g = oracle.layer_split_bwd(p["x"], p, f, p["G"], b, s, heads, 2)
    eps = 1e-6

    def loss(x=None, **over):
        q = dict(p, **over)
        return (oracle.layer_split_fwd(p["x"] if x is None else x, q, b, s, heads, 2, drop=DROP)["x2"] * p["G"]).sum()
    fd = np.zeros_like(p["x"])
    for idx in np.ndindex(p["x"].shape):
        xp, xm = p["x"].copy(), p["x"].copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
    assert _rel(g["dx"], fd) < 1e-7
    # two weights behind dropout sites: the output projection's bias and a QKV weight
    for name, grad, idx in (("bo", g["attn"]["dbo"], (3,)), ("Wqkv", g["attn"]["dWqkv"], (2, 5)),
                            ("b2", g["mlp"]["db2"], (6,))):
        wp, wm = p[name].copy(), p[name].copy()
        wp[idx] += eps
        wm[idx] -= eps
        fdw = (loss(**{name: wp}) - loss(**{name: wm})) / (2 * eps)
        assert abs(grad[idx] - fdw) <= 1e-7 * max(1.0, abs(fdw)), name
