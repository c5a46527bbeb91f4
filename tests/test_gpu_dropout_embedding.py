"""GPU parity of the residual dropout (fused into the partial sums and as a standalone kernel) and
of the vocabulary-parallel embedding, through the C ABI, against the float64 oracle
(oracle/rng.py, oracle/embedding.py).

Keep masks are compared exactly (the kernels' Philox draws must equal the oracle's); values to
rel-L2 <= 1e-6 in fp32 and <= 1e-2 in bf16."""
import numpy as np
import pytest
import torch

import oracle
import oracle.embedding as emb
import oracle.rng as rng
import tp_synth
from tests.gpu_util import dev, dev_i32, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")
TOL = {"f32": 1e-6, "bf16": 1e-2}
TPDT = {"f32": 0, "bf16": 1}


def nonzero(shape, seed, dtype):
    x = tp_synth.normal(seed, 1, shape, 1.0, dtype)
    x[x == 0] = 1.0
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_apply(dtype, p):
    T, n = 333, 264
    x = nonzero((T, n), 41, dtype)
    d = tp.dropout(p, seed=0xDEADBEEF12345, stream=7)
    y = empty((T, n), dtype)
    say(f"[drop] apply {dtype} p={p}")
    tp.tp_dropout_apply(T, n, TPDT[dtype], dev(x, dtype), y, d)
    got = host(y)
    keep = rng.residual_keep(T, n, p, 0xDEADBEEF12345, 7)
    assert np.array_equal(got != 0, keep)
    assert within(rel_l2(got, rng.dropout_apply(x, keep, p)), TOL[dtype])
    # in place gives the same bits
    xi = dev(x, dtype)
    tp.tp_dropout_apply(T, n, TPDT[dtype], xi, xi, d)
    assert np.array_equal(host(xi), got)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dropout_colsum(dtype):
    T, n, p = 1000, 136, 0.25
    x = nonzero((T, n), 42, dtype)
    d = tp.dropout(p, seed=77, stream=5)
    y, cs = empty((T, n), dtype), empty((n,), dtype)
    nb = tp.tp_colsum_workspace(T, n, TPDT[dtype])
    say(f"[drop] dropout+colsum {dtype}")
    tp.tp_dropout_colsum(T, n, TPDT[dtype], dev(x, dtype), y, d, cs, 0, ws(nb), nb)
    keep = rng.residual_keep(T, n, p, 77, 5)
    ref = rng.dropout_apply(x, keep, p)
    got = host(y)
    assert np.array_equal(got != 0, keep)
    assert within(rel_l2(got, ref), TOL[dtype])
    assert within(rel_l2(host(cs), ref.sum(axis=0)), TOL[dtype])
    # accumulate, in place
    base = tp_synth.normal(43, 1, (n,), 1.0, dtype)
    cs2, xi = dev(base, dtype), dev(x, dtype)
    tp.tp_dropout_colsum(T, n, TPDT[dtype], xi, xi, d, cs2, 1, ws(nb), nb)
    assert np.array_equal(host(xi), got)
    assert within(rel_l2(host(cs2), ref.sum(axis=0) + base), TOL[dtype])


def test_dropout_full_size_mask():
    """The 8.3B activation [8192, 3072]: every keep bit against the oracle's generator."""
    T, n, p = 8192, 3072, 0.1
    ones = torch.ones((T, n), dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(ones)
    say("[drop] full-size residual mask")
    tp.tp_dropout_apply(T, n, tp.TP_F32, ones, y, tp.dropout(p, seed=1234, stream=1))
    got = (host(y) != 0)
    assert np.array_equal(got, rng.residual_keep(T, n, p, 1234, 1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sum_partials_with_dropout(dtype):
    rows, cols, t, p = 257, 136, 3, 0.3
    parts = [tp_synth.normal(50 + r, 1, (rows, cols), 1.0, dtype) for r in range(t)]
    bias = tp_synth.normal(60, 1, (cols,), 0.5, dtype)
    res = tp_synth.normal(61, 1, (rows, cols), 1.0, dtype)
    out = empty((rows, cols), dtype)
    d = tp.dropout(p, seed=99, stream=2)
    say(f"[drop] sum_partials {dtype}")
    tp.tp_sum_partials(rows, cols, t, TPDT[dtype], [dev(q, dtype) for q in parts], dev(bias, dtype), dev(res, dtype),
                       out, TPDT[dtype], d)
    keep = rng.residual_keep(rows, cols, p, 99, 2)
    ref = res + rng.dropout_apply(sum(parts) + bias, keep, p)
    assert within(rel_l2(host(out), ref), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sum_partials_layernorm_with_dropout(dtype):
    T, h, t, p = 130, 520, 2, 0.2
    parts = [tp_synth.normal(70 + r, 1, (T, h), 1.0, dtype) for r in range(t)]
    bias = tp_synth.normal(80, 1, (h,), 0.5, dtype)
    res = tp_synth.normal(81, 1, (T, h), 1.0, dtype)
    g = tp_synth.normal(82, 1, (h,), 1.0, dtype)
    b = tp_synth.normal(83, 1, (h,), 0.1, dtype)
    out, y = empty((T, h), dtype), empty((T, h), dtype)
    d = tp.dropout(p, seed=5, stream=11)
    say(f"[drop] sum_partials_layernorm {dtype}")
    tp.tp_sum_partials_layernorm(T, h, t, TPDT[dtype], [dev(q, dtype) for q in parts], dev(bias, dtype),
                                 dev(res, dtype), out, 1e-5, dev(g, dtype), dev(b, dtype), y, None, None, d)
    keep = rng.residual_keep(T, h, p, 5, 11)
    ref = res + rng.dropout_apply(sum(parts) + bias, keep, p)
    got = host(out)
    assert within(rel_l2(got, ref), TOL[dtype])
    # y is LayerNorm of the stored out
    assert within(rel_l2(host(y), oracle.layernorm_fwd(got, g, b)["y"]), TOL[dtype])


def ids_case(seed, N, Vpad):
    g = np.random.default_rng(seed)
    ids = g.integers(0, Vpad, N).astype(np.int32)
    ids[g.random(N) < 0.3] = 5                  # a hot token: long segments across chunks
    ids[:6] = [0, Vpad - 1, Vpad // 4 - 1, Vpad // 4, -3, Vpad + 2]   # boundaries and out-of-range ids
    return ids


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embedding_fwd_bwd(dtype):
    N, h, Vpad, t = 1000, 264, 256, 4
    Vt = Vpad // t
    ids = ids_case(90, N, Vpad)
    E = tp_synth.normal(91, 1, (Vpad, h), 1.0, dtype)
    G = tp_synth.normal(92, 1, (N, h), 1.0, dtype)
    valid = (ids >= 0) & (ids < Vpad)
    total = np.zeros((N, h))
    say(f"[emb] fwd/bwd {dtype}")
    for r in range(t):
        out = empty((N, h), dtype)
        tp.tp_embedding_shard_fwd(N, h, Vpad, t, r, TPDT[dtype], dev_i32(ids), dev(E[r * Vt:(r + 1) * Vt], dtype), out)
        part = host(out)
        assert np.array_equal(part, emb.embed_shard_fwd(ids, E[r * Vt:(r + 1) * Vt], r))
        total += part
        nb = tp.tp_embedding_shard_bwd_workspace(N, Vpad, t)
        dE = empty((Vt, h), dtype)
        w = ws(nb)
        tp.tp_embedding_shard_bwd(N, h, Vpad, t, r, TPDT[dtype], dev_i32(ids), dev(G, dtype), dE, 0, w, nb)
        got = host(dE)
        ref = emb.embed_shard_bwd(ids, G, Vt, r)
        assert within(rel_l2(got, ref), TOL[dtype]), r
        # rows without tokens are exactly zero; repeated calls give identical bits
        assert not got[~ref.any(axis=1)].any()
        dE2 = empty((Vt, h), dtype)
        tp.tp_embedding_shard_bwd(N, h, Vpad, t, r, TPDT[dtype], dev_i32(ids), dev(G, dtype), dE2, 0, w, nb)
        assert np.array_equal(host(dE2), got)
        # accumulate onto an existing gradient
        base = tp_synth.normal(93 + r, 1, (Vt, h), 1.0, dtype)
        dE3 = dev(base, dtype)
        tp.tp_embedding_shard_bwd(N, h, Vpad, t, r, TPDT[dtype], dev_i32(ids), dev(G, dtype), dE3, 1, w, nb)
        assert within(rel_l2(host(dE3), ref + base), TOL[dtype])
    assert np.array_equal(total[valid], E[ids[valid]])
    assert not total[~valid].any()


def test_embedding_empty_and_full_size():
    say("[emb] zero tokens")
    h, Vpad, t = 64, 128, 2
    dE = dev(np.ones((64, h)), "bf16")
    nb = tp.tp_embedding_shard_bwd_workspace(0, Vpad, t)
    tp.tp_embedding_shard_bwd(0, h, Vpad, t, 1, tp.TP_BF16, None, None, dE, 0, ws(nb), nb)
    assert not host(dE).any()
    # 8.3B shape: 8192 tokens, h = 3072, vocabulary 51,200 over 8 ranks; sampled rows
    N, h, Vpad, t, r = 8192, 3072, 51200, 8, 3
    Vt = Vpad // t
    say("[emb] full size rank 3")
    g = np.random.default_rng(94)
    ids = g.integers(0, Vpad, N).astype(np.int32)
    ids[g.random(N) < 0.05] = r * Vt + 17        # a frequent token owned by this rank
    E_r = tp_synth.normal(95, 1, (Vt, h), 1.0, "bf16")
    G = tp_synth.normal(96, 1, (N, h), 1.0, "bf16")
    out = empty((N, h), "bf16")
    tp.tp_embedding_shard_fwd(N, h, Vpad, t, r, tp.TP_BF16, dev_i32(ids), dev(E_r, "bf16"), out)
    assert np.array_equal(host(out), emb.embed_shard_fwd(ids, E_r, r))
    nb = tp.tp_embedding_shard_bwd_workspace(N, Vpad, t)
    dE = empty((Vt, h), "bf16")
    tp.tp_embedding_shard_bwd(N, h, Vpad, t, r, tp.TP_BF16, dev_i32(ids), dev(G, "bf16"), dE, 0, ws(nb), nb)
    got = host(dE)
    rows = np.concatenate([[17], g.choice(Vt, 200, replace=False)])
    for v in rows:
        sel = ids == r * Vt + v
        ref = G[sel].sum(axis=0)
        if sel.any():
            assert within(rel_l2(got[v], ref), 1e-2), v
        else:
            assert not got[v].any(), v
