"""Pins of the oracle's GeLU and MLP block against what the pages and the mathematics fix.

Each test names what it would catch. Nothing here runs on a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


def test_gelu_printed_values():
    """"Megatron-LM, annotated" §2.2 prints GELU(1), GELU(-1), GELU(2) (and §3.1 implies
    GELU(-2)). A wrong form (tanh) or a wrong constant fails at x = 2 or -2."""
    rows = [l.split() for l in open(os.path.join(GOLD, "gelu_printed.txt")) if l.strip() and l[0] != "#"]
    for x, want in rows:
        x, want = float(x), float(want)
        assert round(float(oracle.gelu(x)), 3) == want
        assert round(oracle.gelu_scalar(x), 3) == want


def test_gelu_printed_values_separate_erf_from_tanh():
    """The pin is discriminating: the tanh approximation rounds GELU(2) to 1.955."""
    x = 2.0
    tanh_form = 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert round(tanh_form, 3) != 1.954
    assert round(float(oracle.gelu(x)), 3) == 1.954


def test_gelu_matches_torch_exact_form():
    x = _rng(1).standard_normal(4096) * 4
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(oracle.gelu(x) - ref)) < 1e-14


def test_gelu_grad_autograd_and_fd():
    x = _rng(2).standard_normal(512) * 3
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    torch.nn.functional.gelu(xt).sum().backward()
    assert np.max(np.abs(oracle.gelu_grad(x) - xt.grad.numpy())) < 1e-13
    eps = 1e-6
    fd = (oracle.gelu(x + eps) - oracle.gelu(x - eps)) / (2 * eps)
    assert np.max(np.abs(oracle.gelu_grad(x) - fd)) < 1e-8
    # limits: identity far right, zero far left
    assert abs(float(oracle.gelu_grad(12.0)) - 1.0) < 1e-12
    assert abs(float(oracle.gelu_grad(-12.0))) < 1e-12


def test_mlp_two_by_two_worked_example():
    """"Megatron-LM, annotated" §3.1: the column cut reproduces GELU(XA) locally, the row cut
    with GeLU before the sum gives the printed wrong answer, and the row-parallel second
    matrix gives the printed partials and their sum."""
    g = json.load(open(os.path.join(GOLD, "mlp_cuts_2x2.json")))
    dec = g["decimals"]
    X = np.array([g["X"]], dtype=np.float64)
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    z1, z2 = np.zeros(2), np.zeros(2)
    full = oracle.mlp_fwd(X, A, z1, B, z2)
    assert np.array_equal(full["U"][0], g["XA"])
    assert np.array_equal(np.round(full["Y"][0], dec), g["gelu_XA"])
    # column cut, t = 2: each rank owns one hidden unit
    cols = [oracle.mlp_shard_fwd(X, oracle.shard_cols(A, 2, r), np.zeros(1), oracle.shard_rows(B, 2, r))
            for r in range(2)]
    assert np.array_equal(np.round([c["Y"][0, 0] for c in cols], dec), g["column_cut_outputs"])
    # the row-parallel second matrix: partial sums and their all-reduce
    for r in range(2):
        assert np.array_equal(np.round(cols[r]["Z"][0], dec) + 0.0, g["second_matrix_partials"][r])
    split = oracle.mlp_split_fwd(X, A, z1, B, z2, 2)
    assert np.array_equal(np.round(split["Z"][0], dec), g["second_matrix_sum"])
    assert np.allclose(split["Z"], full["Z"], rtol=0, atol=1e-15)
    # negative control: rows of A, GeLU applied to each partial before adding
    parts = [X[:, i:i + 1] @ A[i:i + 1] for i in range(2)]
    assert np.array_equal(parts[0][0], g["row_cut_partials"][0])
    assert np.array_equal(parts[1][0], g["row_cut_partials"][1])
    wrong = oracle.gelu(parts[0]) + oracle.gelu(parts[1])
    assert np.array_equal(np.round(wrong[0], dec), g["row_cut_gelu_then_add_wrong"])
    assert not np.allclose(wrong, full["Y"])


def _mlp_case(T=16, h=24, ffn=64, seed=3, bias=True):
    g = _rng(seed)
    X = g.standard_normal((T, h))
    A = g.standard_normal((h, ffn)) * 0.3
    B = g.standard_normal((ffn, h)) * 0.3
    b1 = g.standard_normal(ffn) * (0.5 if bias else 0.0)
    b2 = g.standard_normal(h) * (0.5 if bias else 0.0)
    G = g.standard_normal((T, h))
    return X, A, b1, B, b2, G


@pytest.mark.parametrize("t", [1, 2, 4, 8])
def test_mlp_split_equals_unsplit(t):
    """"Tensor and pipeline parallelism..." §3 Proposition: the split is an exact regrouping
    (split equals unsplit to ~1e-15 in float64). Also the per-rank dX_0 is not dX while
    their sum is (the lesson's "In code" checks)."""
    X, A, b1, B, b2, G = _mlp_case()
    full = oracle.mlp_fwd(X, A, b1, B, b2)
    sp = oracle.mlp_split_fwd(X, A, b1, B, b2, t)
    assert _rel(sp["Z"], full["Z"]) < 1e-13
    gf = oracle.mlp_bwd(X, A, B, full["U"], full["Y"], G)
    gs = oracle.mlp_split_bwd(X, A, B, sp["ranks"], G, t)
    for k in ("dX", "dA", "db1", "dB", "db2"):
        assert _rel(gs[k], gf[k]) < 1e-13, k
    if t > 1:
        assert _rel(gs["ranks"][0]["dX"], gf["dX"]) > 1e-3


def test_mlp_backward_against_torch_autograd():
    X, A, b1, B, b2, G = _mlp_case(seed=4)
    tt = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (X, A, b1, B, b2)]
    Z = torch.nn.functional.gelu(tt[0] @ tt[1] + tt[2]) @ tt[3] + tt[4]
    (Z * torch.from_numpy(G)).sum().backward()
    fwd = oracle.mlp_fwd(X, A, b1, B, b2)
    assert _rel(fwd["Z"], Z.detach().numpy()) < 1e-14
    gr = oracle.mlp_bwd(X, A, B, fwd["U"], fwd["Y"], G)
    for k, tv in zip(("dX", "dA", "db1", "dB", "db2"), tt):
        assert _rel(gr[k], tv.grad.numpy()) < 1e-13, k


def test_mlp_backward_finite_differences():
    """Tiny MLP (T=4, h=8, as in the lesson's "In code" cell, t=2): central differences of
    L = sum(G * Z) against every analytic gradient, element by element."""
    X, A, b1, B, b2, G = _mlp_case(T=4, h=8, ffn=32, seed=5)
    t = 2

    def loss(X, A, b1, B, b2):
        return float((oracle.mlp_split_fwd(X, A, b1, B, b2, t)["Z"] * G).sum())

    sp = oracle.mlp_split_fwd(X, A, b1, B, b2, t)
    gs = oracle.mlp_split_bwd(X, A, B, sp["ranks"], G, t)
    args = [X, A, b1, B, b2]
    names = ["dX", "dA", "db1", "dB", "db2"]
    eps = 1e-6
    for i, (arr, name) in enumerate(zip(args, names)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = [a.copy() for a in args]
            m = [a.copy() for a in args]
            p[i][idx] += eps
            m[i][idx] -= eps
            fd[idx] = (loss(*p) - loss(*m)) / (2 * eps)
        assert _rel(gs[name], fd) < 1e-7, name
