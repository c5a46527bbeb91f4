"""GPU parity of the MLP shard (column-parallel GEMM + bias + GeLU, row-parallel partial, and the
backward) against the float64 oracle, through the C ABI. All t ranks run on one device and their
partials are summed on the device (standing in for g forward and f backward).

Tolerances: relative L2 <= 1e-5 for fp32, <= 1e-2 for bf16 (fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import tp_synth
from tests.gpu_util import TP_DT, dev, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")

TOL = {"f32": 1e-5, "bf16": 1e-2}


def run_mlp_ranks(inp, t, dtype, accumulate_into=None):
    """All ranks' fwd + bwd on the device; returns per-rank outputs and the device sums."""
    T, h = inp["X"].shape
    ffn = inp["A"].shape[1]
    Ft = ffn // t
    dt = TP_DT[dtype]
    X, G = dev(inp["X"], dtype), dev(inp["G"], dtype)
    b2 = dev(inp["b2"], "f32")
    ranks = []
    for r in range(t):
        A_r = dev(inp["A"][:, r * Ft:(r + 1) * Ft], dtype)
        b1_r = dev(inp["b1"][r * Ft:(r + 1) * Ft], dtype)
        B_r = dev(inp["B"][r * Ft:(r + 1) * Ft], dtype)
        U, Y, Z = empty((T, Ft), dtype), empty((T, Ft), dtype), empty((T, h), dtype)
        tp.tp_mlp_shard_fwd(T, h, ffn, t, r, dt, X, A_r, b1_r, B_r, U, Y, Z)
        dX, dA, db1, dB = empty((T, h), dtype), empty((h, Ft), dtype), empty((Ft,), dtype), empty((Ft, h), dtype)
        acc = 0
        if accumulate_into is not None:
            dA.copy_(accumulate_into["dA"][r]); db1.copy_(accumulate_into["db1"][r]); dB.copy_(accumulate_into["dB"][r])
            acc = 1
        nbytes = tp.tp_mlp_shard_bwd_workspace(T, h, ffn, t, dt)
        w = ws(nbytes)
        tp.tp_mlp_shard_bwd(T, h, ffn, t, r, dt, X, A_r, B_r, U, Y, G, dX, dA, db1, dB, acc, w, nbytes)
        ranks.append(dict(U=U, Y=Y, Z=Z, dX=dX, dA=dA, db1=db1, dB=dB))
    Zs = empty((T, h), "f32")
    tp.tp_sum_partials(T, h, t, dt, [p["Z"] for p in ranks], b2, None, Zs, tp.TP_F32)
    dXs = empty((T, h), "f32")
    tp.tp_sum_partials(T, h, t, dt, [p["dX"] for p in ranks], None, None, dXs, tp.TP_F32)
    db2 = empty((h,), "f32")
    nb = tp.tp_colsum_workspace(T, h, tp.TP_F32)
    Gf = G.float()
    tp.tp_colsum(T, h, tp.TP_F32, Gf, db2, 0, ws(nb), nb)
    return ranks, {"Z": Zs, "dX": dXs, "db2": db2}


def check_mlp(inp, t, dtype, label):
    say(f"[mlp] {label}: T={inp['X'].shape[0]} h={inp['X'].shape[1]} ffn={inp['A'].shape[1]} t={t} {dtype}")
    ranks, sums = run_mlp_ranks(inp, t, dtype)
    ref = oracle.mlp_fwd(inp["X"], inp["A"], inp["b1"], inp["B"], inp["b2"])
    g = oracle.mlp_bwd(inp["X"], inp["A"], inp["B"], ref["U"], ref["Y"], inp["G"])
    tol = TOL[dtype]
    got = {
        "U": np.concatenate([host(p["U"]) for p in ranks], axis=1),
        "Y": np.concatenate([host(p["Y"]) for p in ranks], axis=1),
        "Z": host(sums["Z"]), "dX": host(sums["dX"]), "db2": host(sums["db2"]),
        "dA": np.concatenate([host(p["dA"]) for p in ranks], axis=1),
        "db1": np.concatenate([host(p["db1"]) for p in ranks]),
        "dB": np.concatenate([host(p["dB"]) for p in ranks], axis=0),
    }
    want = {"U": ref["U"], "Y": ref["Y"], "Z": ref["Z"], **{k: g[k] for k in ("dX", "dA", "db1", "dB", "db2")}}
    errs = {k: rel_l2(got[k], want[k]) for k in want}
    say(f"[mlp] {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, tol), (label, k, e)
    return ranks, sums


def test_mlp_fp32_workload_t2():
    """The fp32 MLP workload: T=128, h=256, ffn=1024, t=2, zero biases."""
    w = tp_synth.WORKLOADS["mlp_fp32_t2"]
    inp = tp_synth.mlp_inputs(w.seed, w.T, w.h, w.ffn, "f32")
    check_mlp(inp, w.t, "f32", "fp32 workload")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_ragged_with_biases(dtype):
    """Sizes that are not multiples of any tile (T=200, h=136, F/t=296) and nonzero biases."""
    inp = tp_synth.mlp_inputs(77, 200, 136, 592, dtype, bias_std=0.5)
    check_mlp(inp, 2, dtype, f"ragged {dtype}")


def test_mlp_bf16_multitile_t4():
    inp = tp_synth.mlp_inputs(78, 1024, 512, 2048, "bf16", bias_std=0.1)
    check_mlp(inp, 4, "bf16", "multi-tile t=4")


def test_mlp_bf16_long_k_split():
    """Tall-skinny weight gradients (K = T = 4096 tokens) go through split-K."""
    inp = tp_synth.mlp_inputs(79, 4096, 256, 512, "bf16")
    check_mlp(inp, 2, "bf16", "long-K wgrad")


def test_mlp_deterministic_and_accumulate():
    inp = tp_synth.mlp_inputs(80, 256, 128, 512, "bf16", bias_std=0.2)
    r1, s1 = run_mlp_ranks(inp, 2, "bf16")
    r2, s2 = run_mlp_ranks(inp, 2, "bf16")
    for k in ("U", "Y", "Z", "dX", "dA", "db1", "dB"):
        for a, b in zip(r1, r2):
            assert torch.equal(a[k], b[k]), k
    # accumulate=1 adds the new gradients into the old ones
    prev = {k: [p[k].clone() for p in r1] for k in ("dA", "db1", "dB")}
    r3, _ = run_mlp_ranks(inp, 2, "bf16", accumulate_into=prev)
    for k in ("dA", "db1", "dB"):
        for a, b in zip(r3, r1):
            assert rel_l2(host(a[k]), 2 * host(b[k])) < 1e-2, k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_zero_tokens(dtype):
    """T = 0: the forward launches nothing; the weight gradients are zero."""
    h, ffn, t = 64, 256, 2
    Ft = ffn // t
    dt = TP_DT[dtype]
    X, G = empty((0, h), dtype), empty((0, h), dtype)
    A_r, B_r = dev(np.ones((h, Ft)), dtype), dev(np.ones((Ft, h)), dtype)
    U, Y, Z = empty((0, Ft), dtype), empty((0, Ft), dtype), empty((0, h), dtype)
    # empty tensors have no storage: pass aligned dummies
    dummy = empty((64,), dtype)
    tp.tp_mlp_shard_fwd(0, h, ffn, t, 0, dt, dummy, A_r, None, B_r, dummy, dummy, dummy)
    dA, db1, dB = dev(np.full((h, Ft), 3.0), dtype), dev(np.full(Ft, 3.0), dtype), dev(np.full((Ft, h), 3.0), dtype)
    nbytes = tp.tp_mlp_shard_bwd_workspace(0, h, ffn, t, dt)
    tp.tp_mlp_shard_bwd(0, h, ffn, t, 0, dt, dummy, A_r, B_r, dummy, dummy, dummy, dummy, dA, db1, dB, 0,
                        ws(nbytes), nbytes)
    for x in (dA, db1, dB):
        assert np.all(host(x) == 0)


def test_mlp_8p3b_shape_rank0_sampled():
    """The 8.3B shard shape (T=8192, h=3072, F/t=1536, rank 0 of t=8): every output checked on
    sampled rows (forward, dX) and sampled columns/rows (dA, db1, dB) computed one by one in
    float64."""
    T, h, ffn, t, r = 8192, 3072, 12288, 8, 0
    Ft = ffn // t
    w = tp_synth.WORKLOADS["layer_8p3b_t8"]
    rng = np.random.default_rng([w.seed, 99])
    X = tp_synth.normal(w.seed, 0, (T, h), 1.0, "bf16")
    G = tp_synth.normal(w.seed, 1, (T, h), 1.0, "bf16")
    A_r = tp_synth.normal(w.seed, 2, (h, Ft), 0.02, "bf16")
    B_r = tp_synth.normal(w.seed, 3, (Ft, h), 0.02, "bf16")
    say("[mlp] 8.3B shard shape, rank 0")
    dt = tp.TP_BF16
    Xd, Gd, Ad, Bd = dev(X, "bf16"), dev(G, "bf16"), dev(A_r, "bf16"), dev(B_r, "bf16")
    U, Y, Z = empty((T, Ft), "bf16"), empty((T, Ft), "bf16"), empty((T, h), "bf16")
    tp.tp_mlp_shard_fwd(T, h, ffn, t, r, dt, Xd, Ad, None, Bd, U, Y, Z)
    dX, dA, db1, dB = empty((T, h), "bf16"), empty((h, Ft), "bf16"), empty((Ft,), "bf16"), empty((Ft, h), "bf16")
    nb = tp.tp_mlp_shard_bwd_workspace(T, h, ffn, t, dt)
    tp.tp_mlp_shard_bwd(T, h, ffn, t, r, dt, Xd, Ad, Bd, U, Y, Gd, dX, dA, db1, dB, 0, ws(nb), nb)
    rows = np.sort(rng.choice(T, 48, replace=False))
    cols = np.sort(rng.choice(Ft, 24, replace=False))
    # forward and dX on sampled token rows (each row depends only on its own token)
    f = oracle.mlp_shard_fwd(X[rows], A_r, np.zeros(Ft), B_r)
    bw = oracle.mlp_shard_bwd(X[rows], A_r, B_r, f["U"], f["Y"], G[rows])
    errs = {"U": rel_l2(host(U)[rows], f["U"]), "Y": rel_l2(host(Y)[rows], f["Y"]),
            "Z": rel_l2(host(Z)[rows], f["Z"]), "dX": rel_l2(host(dX)[rows], bw["dX"])}
    # dA[:, j] = X^T dU[:, j], dU[:, j] = (G B_r[j]^T) * GeLU'(X A_r[:, j]); db1[j] = sum dU[:, j]
    Uc = X @ A_r[:, cols]
    dUc = (G @ B_r[cols].T) * oracle.gelu_grad(Uc)
    errs["dA"] = rel_l2(host(dA)[:, cols], X.T @ dUc)
    errs["db1"] = rel_l2(host(db1)[cols], dUc.sum(axis=0))
    # dB[i, :] = Y[:, i]^T G
    ib = cols[:8]
    errs["dB"] = rel_l2(host(dB)[ib], oracle.gelu(X @ A_r[:, ib]).T @ G)
    say("[mlp] 8.3B rank 0: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, 1e-2), (k, e)
