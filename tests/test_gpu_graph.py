"""The layer step captured into a HIP graph and replayed: every replay must reproduce the eager
step bit for bit (the library launches only kernels, all on the caller's stream: no
allocation, no memset, no synchronisation, no stream or event of its own), with
eager work and synchronisations between the replays. Dropout is on, so the Philox draws and the
attention keep-bit mask run under capture too."""
import numpy as np
import pytest
import torch

import tp_synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")
from tensor_transformer_layer_amd.layer import LayerShard, rank_params  # noqa: E402
from tests.test_gpu_layer import DROP, rank_drop  # noqa: E402

NAMES = ("x2", "dx", "dA", "db1", "dB", "db2", "dWqkv", "dbqkv", "dWo", "dbo", "dln1_g", "dln1_b", "dln2_g",
         "dln2_b", "x1", "QKV", "O", "lse", "U", "Y")


@pytest.mark.parametrize("recompute", [False, True])
def test_layer_step_graph_replay_matches_eager(recompute):
    b, s, h, heads, ffn, t = 2, 128, 256, 4, 1024, 2
    dev = "cuda:0"
    p = tp_synth.layer_inputs(4747, b, s, h, ffn, "bf16", bias_std=0.05, ln_random=True)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)

    x, G = d(p["x"]), d(p["G"])
    T = b * s
    g = np.random.default_rng(4748)
    sums = [d(g.standard_normal((T, h)).astype(np.float32)) for _ in range(4)]   # the four all-reduce results
    sh = LayerShard(b, s, h, heads, ffn, t, 0, rank_params(p, heads, t, 0, dev), dev, rank_drop(DROP, 0))
    sh.step(x, G, *sums, recompute=recompute)
    torch.cuda.synchronize()
    eager = {k: getattr(sh, k).clone() for k in NAMES}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on a side stream before capture
        sh.step(x, G, *sums, recompute=recompute)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sh.step(x, G, *sums, recompute=recompute)
    for rep in range(3):
        for k in NAMES:                     # clobber every output between replays (eager work)
            getattr(sh, k).fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {rep} recompute={recompute}")
        for k in NAMES:
            assert torch.equal(getattr(sh, k), eager[k]), (rep, k)


_FIRST_CALL_UNDER_CAPTURE = r"""
import numpy as np, torch, sys
sys.path[:0] = sys.argv[1:]
import tp_synth
from tensor_transformer_layer_amd.layer import LayerShard, rank_params
from tests.test_gpu_layer import DROP, rank_drop
b, s, h, heads, ffn, t = 2, 128, 256, 4, 1024, 2
dev = "cuda:0"
p = tp_synth.layer_inputs(4749, b, s, h, ffn, "bf16", bias_std=0.05, ln_random=True)
d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).to(dev)
x, G = d(p["x"]), d(p["G"])
g = np.random.default_rng(4750)
sums = [d(g.standard_normal((b * s, h)).astype(np.float32)) for _ in range(4)]
sh = LayerShard(b, s, h, heads, ffn, t, 0, rank_params(p, heads, t, 0, dev), dev, rank_drop(DROP, 0))
sh.attn_fwd(x)                 # forward kernels only: no backward call has run in this process
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):  # the first backward calls come under capture
    sh.step(x, G, *sums)
graph.replay()
torch.cuda.synchronize()
names = %r
got = {k: getattr(sh, k).clone() for k in names}
sh.step(x, G, *sums)           # eager, after the replay
torch.cuda.synchronize()
bad = [k for k in names if not torch.equal(getattr(sh, k), got[k])]
print("mismatch:", bad, flush=True)
sys.exit(1 if bad else 0)
""" % (NAMES,)


def test_first_backward_call_under_capture():
    """A process whose first backward call is made while its stream is being captured: the
    library keeps no per-process state that a first call would have to create, so the replay
    equals the eager step run afterwards. Fresh process, so that no earlier call has run."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("[graph] first backward call under capture (child process)")
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_UNDER_CAPTURE, root, os.path.join(root, "tests")],
                       capture_output=True, text=True, timeout=240, cwd=root)
    say(r.stdout[-2000:] + r.stderr[-2000:])
    assert r.returncode == 0
