"""GPU check of tp_vocab_xent_shard_fwd_noalloc, the allocation-free form of the fused vocabulary
logits + cross-entropy statistics call: its per-(tile, token) partials live in the library's own
scratch array instead of a caller workspace. Two calls in a row, the second on a smaller input, each
compared with the workspace form (tp_vocab_xent_shard_fwd) on the same inputs: the same kernels in
the same order, so max, sum of exponentials, target logit and argmax must be equal bit for bit;
the statistics are also held to the float64 oracle (relative L2 1e-2 with the element and row
bounds). A shape beyond the scratch is refused."""
import numpy as np
import pytest
import torch

import oracle
import tp_synth
from tests.gpu_util import dev, dev_i32, empty, host, rel_l2, say, within, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")


def both_forms(inp, N, h, Vpad, Vreal, t, r, mask):
    X, tg = dev(inp["X"], "bf16"), dev_i32(inp["targets"])
    Vt = Vpad // t
    E_r = dev(inp["E"][r * Vt:(r + 1) * Vt], "bf16")
    outs = []
    for form in ("workspace", "noalloc"):
        mx, se, tv = empty((N,), "f32"), empty((N,), "f32"), empty((N,), "f32")
        am = torch.full((N,), -1, dtype=torch.int32, device="cuda:0")
        if form == "workspace":
            nb = tp.tp_vocab_xent_shard_fwd_workspace(N, h, Vpad, t, tp.TP_BF16)
            tp.tp_vocab_xent_shard_fwd(N, h, Vpad, Vreal, t, r, tp.TP_BF16, mask, X, E_r, tg, mx, se, tv, am, ws(nb), nb)
        else:
            tp.tp_vocab_xent_shard_fwd_noalloc(N, h, Vpad, Vreal, t, r, tp.TP_BF16, mask, X, E_r, tg, mx, se, tv, am)
        torch.cuda.synchronize()
        outs.append({"max": mx, "sumexp": se, "tgt": tv, "argmax": am})
    return outs


@pytest.mark.parametrize("label,seed,N,h,Vreal,Vpad,t,r,mask", [
    # two launches (256x256 and 64x64 tiles), 28 tile rows x 4136 tokens of partials
    ("large, two-part launch", 501, 4136, 520, 8300, 8320, 2, 1, 1),
    # then a smaller call that leaves most of the previous call's partials in the scratch
    ("smaller, after the large one", 502, 300, 200, 1000, 1024, 4, 2, 0),
])
def test_noalloc_matches_workspace_form(label, seed, N, h, Vreal, Vpad, t, r, mask):
    inp = tp_synth.xent_inputs(seed, N, h, Vreal, Vpad, "bf16", e_std=0.2)
    say(f"[noalloc] {label}: N={N} h={h} Vpad={Vpad} t={t} r={r} mask={mask}")
    ref, got = both_forms(inp, N, h, Vpad, Vreal, t, r, mask)
    for k in ("max", "sumexp", "tgt", "argmax"):
        assert torch.equal(got[k], ref[k]), (label, k)
    st = oracle.xent_shard_stats(inp["X"], oracle.vocab_shard(inp["E"], t, r), inp["targets"], t, r, Vreal, bool(mask))
    for k in ("max", "sumexp", "tgt"):
        e = rel_l2(host(got[k]), st[k])
        say(f"[noalloc] {label}: {k} {e!r}")
        assert within(e, 1e-2), (label, k, e)


def test_noalloc_refuses_beyond_scratch():
    N, h, Vpad, t = 65536, 64, 51200, 8
    d = empty((64,), "f32")
    with pytest.raises(tp.TPError, match="scratch"):
        tp.tp_vocab_xent_shard_fwd_noalloc(N, h, Vpad, 50257, t, 0, tp.TP_BF16, 0, d, d, d, d, d, d, d)
