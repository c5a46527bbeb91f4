"""GPU parity of the head-sharded attention shard (QKV projection, causal attention, row-parallel
output projection, and the backward) against the float64 oracle, through the C ABI.

Tolerance: relative L2 <= 1e-2 (bf16 operands, fp32 accumulation and fp32 softmax)."""
import numpy as np
import pytest

import oracle
import tp_synth
from tests.gpu_util import dev, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")

TOL = 1e-2


def run_attn_ranks(inp, b, s, h, heads, t, causal=1, ranks_to_run=None):
    T = b * s
    ht = h // t
    dt = tp.TP_BF16
    Xn, G = dev(inp["Xn"], "bf16"), dev(inp["G"], "bf16")
    out = []
    for r in (ranks_to_run if ranks_to_run is not None else range(t)):
        Wqkv_r = dev(oracle.qkv_shard(inp["Wqkv"], heads, t, r), "bf16")
        bqkv_r = dev(oracle.qkv_shard(inp["bqkv"], heads, t, r), "bf16")
        Wo_r = dev(oracle.wo_shard(inp["Wo"], heads, t, r), "bf16")
        QKV, O, Z = empty((T, 3 * ht), "bf16"), empty((T, ht), "bf16"), empty((T, h), "bf16")
        lse = empty((b, heads // t, s), "f32")
        tp.tp_attn_shard_fwd(b, s, h, heads, t, r, dt, causal, Xn, Wqkv_r, bqkv_r, Wo_r, QKV, O, lse, Z)
        dXn, dWqkv, dbqkv, dWo = empty((T, h), "bf16"), empty((h, 3 * ht), "bf16"), empty((3 * ht,), "bf16"), empty((ht, h), "bf16")
        nb = tp.tp_attn_shard_bwd_workspace(b, s, h, heads, t, dt)
        tp.tp_attn_shard_bwd(b, s, h, heads, t, r, dt, causal, Xn, Wqkv_r, Wo_r, QKV, O, lse, G, dXn, dWqkv, dbqkv,
                             dWo, 0, ws(nb), nb)
        out.append(dict(r=r, QKV=QKV, O=O, lse=lse, Z=Z, dXn=dXn, dWqkv=dWqkv, dbqkv=dbqkv, dWo=dWo))
    return out


def check_attn(inp, b, s, h, heads, t, causal, label):
    say(f"[attn] {label}: b={b} s={s} h={h} heads={heads} t={t} causal={causal}")
    ranks = run_attn_ranks(inp, b, s, h, heads, t, causal)
    T = b * s
    bo = dev(inp["bo"], "f32")
    Zs, dXs = empty((T, h), "f32"), empty((T, h), "f32")
    tp.tp_sum_partials(T, h, t, tp.TP_BF16, [p["Z"] for p in ranks], bo, None, Zs, tp.TP_F32)
    tp.tp_sum_partials(T, h, t, tp.TP_BF16, [p["dXn"] for p in ranks], None, None, dXs, tp.TP_F32)
    f = oracle.attn_split_fwd(inp["Xn"], inp["Wqkv"], inp["bqkv"], inp["Wo"], inp["bo"], b, s, heads, t, causal)
    g = oracle.attn_split_bwd(inp["Xn"], inp["Wqkv"], inp["Wo"], f["ranks"], inp["G"], b, s, heads, t)
    errs = {"Z": rel_l2(host(Zs), f["Z"]), "dXn": rel_l2(host(dXs), g["dXn"])}
    for p in ranks:
        r = p["r"]
        fr, gr = f["ranks"][r], g["ranks"][r]
        for k, want in (("QKV", fr["QKV"]), ("O", fr["O"]), ("lse", fr["lse"]), ("dWqkv", gr["dWqkv"]),
                        ("dbqkv", gr["dbqkv"]), ("dWo", gr["dWo"])):
            errs[f"{k}{r}"] = rel_l2(host(p[k]), want)
    say(f"[attn] {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, TOL), (label, k, e)


@pytest.mark.parametrize("causal", [1, 0])
def test_attn_ragged_small(causal):
    """b=2, s=200 (a ragged 64-row tail), 4 heads of 96, t=2, nonzero biases."""
    b, s, h, heads, t = 2, 200, 384, 4, 2
    inp = tp_synth.attn_inputs(91, b, s, h, "bf16", bias_std=0.2, w_std=0.05)
    check_attn(inp, b, s, h, heads, t, causal, f"ragged causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 192])
def test_attn_other_head_widths(d):
    b, s, heads, t = 1, 256, 4, 2
    h = heads * d
    inp = tp_synth.attn_inputs(92, b, s, h, "bf16", bias_std=0.1, w_std=0.05)
    check_attn(inp, b, s, h, heads, t, 1, f"d={d}")


def test_attn_single_position():
    """s = 1: the only visible key is the query's own, so O = V and lse = the one scaled score."""
    b, s, h, heads, t = 3, 1, 192, 2, 1
    inp = tp_synth.attn_inputs(93, b, s, h, "bf16", bias_std=0.3)
    check_attn(inp, b, s, h, heads, t, 1, "s=1")
    r = run_attn_ranks(inp, b, s, h, heads, t, 1)[0]
    qkv = host(r["QKV"])
    assert np.array_equal(host(r["O"]), qkv[:, 2 * h:3 * h])


def test_attn_deterministic():
    b, s, h, heads, t = 1, 128, 192, 2, 1
    inp = tp_synth.attn_inputs(94, b, s, h, "bf16")
    a = run_attn_ranks(inp, b, s, h, heads, t)[0]
    c = run_attn_ranks(inp, b, s, h, heads, t)[0]
    for k in ("QKV", "O", "lse", "Z", "dXn", "dWqkv", "dbqkv", "dWo"):
        assert bool((a[k] == c[k]).all()), k


def test_attn_accumulate_and_optional_bias_grad():
    """accumulate = 1 adds the new dWqkv, dbqkv and dWo to the old ones (dXn is overwritten); with
    dbqkv = NULL the kernels skip their column sums and every other output is bit-identical."""
    b, s, h, heads, t, r = 2, 200, 384, 4, 2, 1
    inp = tp_synth.attn_inputs(95, b, s, h, "bf16", bias_std=0.2, w_std=0.05)
    T, ht, dt = b * s, h // t, tp.TP_BF16
    Xn, G = dev(inp["Xn"], "bf16"), dev(inp["G"], "bf16")
    Wqkv_r = dev(oracle.qkv_shard(inp["Wqkv"], heads, t, r), "bf16")
    bqkv_r = dev(oracle.qkv_shard(inp["bqkv"], heads, t, r), "bf16")
    Wo_r = dev(oracle.wo_shard(inp["Wo"], heads, t, r), "bf16")
    QKV, O, Z = empty((T, 3 * ht), "bf16"), empty((T, ht), "bf16"), empty((T, h), "bf16")
    lse = empty((b, heads // t, s), "f32")
    tp.tp_attn_shard_fwd(b, s, h, heads, t, r, dt, 1, Xn, Wqkv_r, bqkv_r, Wo_r, QKV, O, lse, Z)
    nb = tp.tp_attn_shard_bwd_workspace(b, s, h, heads, t, dt)

    def bwd(dbqkv, acc, prev=None):
        o = dict(dXn=empty((T, h), "bf16"), dWqkv=empty((h, 3 * ht), "bf16"), dWo=empty((ht, h), "bf16"))
        if prev is not None:
            o["dWqkv"].copy_(prev["dWqkv"]); o["dWo"].copy_(prev["dWo"])
        tp.tp_attn_shard_bwd(b, s, h, heads, t, r, dt, 1, Xn, Wqkv_r, Wo_r, QKV, O, lse, G, o["dXn"], o["dWqkv"],
                             dbqkv, o["dWo"], acc, ws(nb), nb)
        o["dbqkv"] = dbqkv
        return o

    first = bwd(empty((3 * ht,), "bf16"), 0)
    nob = bwd(None, 0)
    for k in ("dXn", "dWqkv", "dWo"):
        assert bool((first[k] == nob[k]).all()), k
    db = first["dbqkv"].clone()
    second = bwd(db, 1, prev=first)
    for k in ("dWqkv", "dWo", "dbqkv"):
        e = rel_l2(host(second[k]), 2 * host(first[k]))
        say(f"[attn] accumulate {k}: {e:.2e}")
        assert e < 1e-2, k
    assert bool((second["dXn"] == first["dXn"]).all())


def _sampled_full_size(w, ranks_to_run, seq, tol=TOL):
    """Full-size shard: the oracle is run on one sequence (every head of the rank) and on one head
    (every sequence), which fixes sampled rows of Z, O, lse, dXn and sampled columns of the weight
    gradients exactly."""
    b, s, h, heads, t = w.b, w.s, w.h, w.heads, w.t
    d = h // heads
    ht = h // t
    hl = heads // t
    inp = tp_synth.attn_inputs(w.seed, b, s, h, "bf16")
    say(f"[attn] full size {w.name}: ranks {list(ranks_to_run)}")
    ranks = run_attn_ranks(inp, b, s, h, heads, t, 1, ranks_to_run)
    rows = slice(seq * s, (seq + 1) * s)
    for p in ranks:
        r = p["r"]
        Wqkv_r = oracle.qkv_shard(inp["Wqkv"], heads, t, r)
        Wo_r = oracle.wo_shard(inp["Wo"], heads, t, r)
        bq = oracle.qkv_shard(inp["bqkv"], heads, t, r)
        # one sequence, all the rank's heads
        f1 = oracle.attn_shard_fwd(inp["Xn"][rows], Wqkv_r, bq, Wo_r, 1, s, hl)
        g1 = oracle.attn_shard_bwd(inp["Xn"][rows], Wqkv_r, Wo_r, f1, inp["G"][rows], 1, s, hl)
        errs = {"QKV": rel_l2(host(p["QKV"])[rows], f1["QKV"]), "O": rel_l2(host(p["O"])[rows], f1["O"]),
                "lse": rel_l2(host(p["lse"])[seq], f1["lse"][0]), "Z": rel_l2(host(p["Z"])[rows], f1["Z"]),
                "dXn": rel_l2(host(p["dXn"])[rows], g1["dXn"])}
        # local head 0 of the rank, every sequence: its Q/K/V columns of dWqkv, dbqkv and its rows of dWo
        cols = np.concatenate([np.arange(i * ht, i * ht + d) for i in range(3)])
        Wh = Wqkv_r[:, cols]
        fh = oracle.attn_shard_fwd(inp["Xn"], Wh, bq[cols], Wo_r[:d], b, s, 1)
        gh = oracle.attn_shard_bwd(inp["Xn"], Wh, Wo_r[:d], fh, inp["G"], b, s, 1)
        errs["dWqkv_h0"] = rel_l2(host(p["dWqkv"])[:, cols], gh["dWqkv"])
        errs["dbqkv_h0"] = rel_l2(host(p["dbqkv"])[cols], gh["dbqkv"])
        errs["dWo_h0"] = rel_l2(host(p["dWo"])[:d], gh["dWo"])
        say(f"[attn] {w.name} rank {r}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, e in errs.items():
            assert within(e, tol), (w.name, r, k, e)


def test_attn_1p2b_workload_full_size():
    """The 1.2B attention workload (b=8, s=1024, h=1536, 16 heads of 96, t=2) in full: both ranks'
    QKV, O, lse, dWqkv, dbqkv and dWo over every sequence and head, and the device sums of the
    two ranks' Z and dXn partials, against the float64 split oracle element by element."""
    w = tp_synth.WORKLOADS["attn_1p2b_t2"]
    inp = tp_synth.attn_inputs(w.seed, w.b, w.s, w.h, "bf16")
    check_attn(inp, w.b, w.s, w.h, w.heads, w.t, 1, "1.2B workload, full size")


def test_attn_8p3b_shard_full_size():
    """The 8.3B layer's attention shard (h=3072, 32 heads, t=8), rank 0 and rank 7."""
    _sampled_full_size(tp_synth.WORKLOADS["layer_8p3b_t8"], [0, 7], seq=2)


@pytest.mark.parametrize("heads", [16, 24])
def test_attn_8p3b_head_sweep_full_size(heads):
    """The pages' 8.3B head-count sweep: the same shard with 16 heads of 192 or 24 heads of 128
    (2 or 3 heads per rank), rank 0 at full size."""
    import dataclasses
    w = dataclasses.replace(tp_synth.WORKLOADS["layer_8p3b_t8"], heads=heads, name=f"layer_8p3b_t8_h{heads}")
    _sampled_full_size(w, [0], seq=3)
