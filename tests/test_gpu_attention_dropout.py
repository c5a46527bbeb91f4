"""GPU parity of attention dropout (per-rank Philox stream, "Megatron-LM ..." digest §3.4, Random
Number Generation Handling) through the C ABI against the float64 oracle: the keep-bit mask the
forward writes (bit-exact for every visible element), and the forward and backward outputs of the
shard with the same masks (rel-L2 <= 1e-2, bf16)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.rng as rng
import tp_synth
from tests.gpu_util import dev, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")
TOL = 1e-2
SEED = 0x5EED0123456789


def stream_of(r):
    return 1000 + r


def mask_bits(mask, b, hl, s):
    """Decode the [b][hl][s][ceil(s/32)] keep words into booleans [b, hl, s, s]."""
    n32 = (s + 31) // 32
    w = mask.cpu().numpy().view(np.uint32)[: b * hl * s * n32].reshape(b, hl, s, n32)
    k = np.arange(s)
    return ((w[..., k // 32] >> (k % 32).astype(np.uint32)) & 1).astype(bool)


def run_rank(inp, b, s, h, heads, t, r, causal, p):
    T, ht, hl = b * s, h // t, heads // t
    Xn, G = dev(inp["Xn"], "bf16"), dev(inp["G"], "bf16")
    Wqkv_r = dev(oracle.qkv_shard(inp["Wqkv"], heads, t, r), "bf16")
    bqkv_r = dev(oracle.qkv_shard(inp["bqkv"], heads, t, r), "bf16")
    Wo_r = dev(oracle.wo_shard(inp["Wo"], heads, t, r), "bf16")
    mask = torch.zeros(tp.tp_attn_dropout_mask_bytes(b, s, heads, t) // 4 + 4, dtype=torch.int32, device="cuda:0")
    d = tp.dropout(p, SEED, stream_of(r), mask)
    QKV, O, Z = empty((T, 3 * ht), "bf16"), empty((T, ht), "bf16"), empty((T, h), "bf16")
    lse = empty((b, hl, s), "f32")
    tp.tp_attn_shard_fwd(b, s, h, heads, t, r, tp.TP_BF16, causal, Xn, Wqkv_r, bqkv_r, Wo_r, QKV, O, lse, Z, d)
    dXn, dWqkv, dbqkv, dWo = empty((T, h), "bf16"), empty((h, 3 * ht), "bf16"), empty((3 * ht,), "bf16"), empty((ht, h), "bf16")
    nb = tp.tp_attn_shard_bwd_workspace(b, s, h, heads, t, tp.TP_BF16)
    tp.tp_attn_shard_bwd(b, s, h, heads, t, r, tp.TP_BF16, causal, Xn, Wqkv_r, Wo_r, QKV, O, lse, G, dXn, dWqkv, dbqkv,
                         dWo, 0, ws(nb), nb, d)
    return dict(mask=mask, O=O, lse=lse, Z=Z, dXn=dXn, dWqkv=dWqkv, dbqkv=dbqkv, dWo=dWo)


def oracle_rank(inp, b, s, h, heads, t, r, causal, p):
    Wqkv_r = oracle.qkv_shard(inp["Wqkv"], heads, t, r)
    Wo_r = oracle.wo_shard(inp["Wo"], heads, t, r)
    bq = oracle.qkv_shard(inp["bqkv"], heads, t, r)
    drop = {"p": p, "seed": SEED, "stream": stream_of(r), "heads": heads, "head0": r * (heads // t)}
    f = oracle.attn_shard_fwd(inp["Xn"], Wqkv_r, bq, Wo_r, b, s, heads // t, bool(causal), drop)
    g = oracle.attn_shard_bwd(inp["Xn"], Wqkv_r, Wo_r, f, inp["G"], b, s, heads // t)
    return f, g


@pytest.mark.parametrize("causal,d,s,p", [(1, 96, 100, 0.2), (0, 96, 100, 0.2), (1, 64, 160, 0.5), (1, 128, 96, 0.1),
                                          (1, 192, 70, 0.3)])
def test_attention_dropout_small(causal, d, s, p):
    b, heads, t = 2, 4, 2
    h = heads * d
    inp = tp_synth.attn_inputs(120 + d + s, b, s, h, "bf16", bias_std=0.2, w_std=0.05)
    hl = heads // t
    vis = np.tril(np.ones((s, s), dtype=bool)) if causal else np.ones((s, s), dtype=bool)
    masks = []
    for r in range(t):
        say(f"[attn-drop] causal={causal} d={d} s={s} p={p} rank {r}")
        got = run_rank(inp, b, s, h, heads, t, r, causal, p)
        f, g = oracle_rank(inp, b, s, h, heads, t, r, causal, p)
        bits = mask_bits(got["mask"], b, hl, s)
        for bi in range(b):
            for j in range(hl):
                assert np.array_equal(bits[bi, j][vis], f["keep"][bi, j][vis]), (r, bi, j)
        masks.append(bits)
        errs = {k: rel_l2(host(got[k]), want) for k, want in
                (("O", f["O"]), ("lse", f["lse"]), ("Z", f["Z"]), ("dXn", g["dXn"]), ("dWqkv", g["dWqkv"]),
                 ("dbqkv", g["dbqkv"]), ("dWo", g["dWo"]))}
        say("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, e in errs.items():
            assert within(e, TOL), (r, k, e)
    # the two ranks draw different patterns (per-rank streams)
    assert 0.3 < (masks[0][0, 0][vis] == masks[1][0, 0][vis]).mean() < 0.95


def test_attention_dropout_full_size_8p3b_rank0():
    """8.3B shard (b=8, s=1024, 32 heads of 96, t=8), rank 0, p=0.1: the mask of sequence 0 (all four
    heads) bit-exact, and sequence 0's outputs against the oracle run on that sequence."""
    b, s, h, heads, t, p = 8, 1024, 3072, 32, 8, 0.1
    hl = heads // t
    inp = tp_synth.attn_inputs(130, b, s, h, "bf16")
    say("[attn-drop] full size 8.3B rank 0")
    got = run_rank(inp, b, s, h, heads, t, 0, 1, p)
    bits = mask_bits(got["mask"], 1, hl, s)    # sequence 0 comes first in the layout
    vis = np.tril(np.ones((s, s), dtype=bool))
    for j in range(hl):
        want = rng.attn_keep(0, j, s, heads, p, SEED, stream_of(0))
        assert np.array_equal(bits[0, j][vis], want[vis]), j
    rows = slice(0, s)
    one = {k: (v[rows] if k in ("Xn", "G") else v) for k, v in inp.items()}
    f, g = oracle_rank(one, 1, s, h, heads, t, 0, 1, p)
    errs = {"O": rel_l2(host(got["O"])[rows], f["O"]), "Z": rel_l2(host(got["Z"])[rows], f["Z"]),
            "dXn": rel_l2(host(got["dXn"])[rows], g["dXn"])}
    say("   " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert within(e, TOL), (k, e)
