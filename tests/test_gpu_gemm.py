"""GPU parity of tp_gemm_bf16, the GEMM the shard calls are built from, through the C ABI: each
operand layout with its epilogues, ragged sizes, split K, K = 0 and accumulate, against float64
products of the same bf16 inputs (numpy matmul as the reference product; GeLU and its derivative
from the oracle). Also: backward calls on two streams at once give the bits of the same calls made
one after the other (the library keeps no state shared between calls).

Tolerance: relative L2 <= 1e-2 (bf16 operands and outputs, fp32 accumulation), with the element
and row bounds of tests/gpu_util.within."""
import numpy as np
import pytest
import torch

import oracle
import tp_synth
from tests.gpu_util import dev, empty, host, rel_l2, say, within, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")


def operands(seed, M, N, K, a_mn, b_mn):
    g = np.random.default_rng(seed)
    A = tp_synth.round_to_dtype(g.standard_normal((M, K)), "bf16")
    B = tp_synth.round_to_dtype(g.standard_normal((K, N)) * 0.05, "bf16")
    Ad = dev(A.T if a_mn else A, "bf16")          # (m, k) at [k, m] when MN-contiguous
    Bd = dev(B if b_mn else B.T, "bf16")          # (k, n) at [k, n] when MN-contiguous
    return A, B, Ad, Bd


@pytest.mark.parametrize("M,N,K", [(200, 136, 72), (1000, 520, 264), (296, 1024, 4096)])
@pytest.mark.parametrize("a_mn,b_mn", [(0, 0), (0, 1), (1, 1)])
def test_gemm_layouts_store(M, N, K, a_mn, b_mn):
    A, B, Ad, Bd = operands(M * 7 + N + K + 31 * a_mn + 17 * b_mn, M, N, K, a_mn, b_mn)
    g = np.random.default_rng(5)
    bias = tp_synth.round_to_dtype(g.standard_normal(N), "bf16")
    C = empty((M, N), "bf16")
    nb = tp.tp_gemm_bf16_workspace(M, N, K)
    lda, ldb = (M if a_mn else K), (N if b_mn else K)
    tp.tp_gemm_bf16(M, N, K, Ad, lda, a_mn, Bd, ldb, b_mn, tp.TP_EPI_STORE, C, None, N, dev(bias, "bf16"), None, 0,
                    ws(nb), nb)
    e = rel_l2(host(C), A @ B + bias)
    say(f"[gemm] {M}x{N}x{K} a_mn={a_mn} b_mn={b_mn} store+bias: {e!r}")
    assert within(e, 1e-2)
    # accumulate onto the result: C + P
    C0 = host(C)
    tp.tp_gemm_bf16(M, N, K, Ad, lda, a_mn, Bd, ldb, b_mn, tp.TP_EPI_STORE, C, None, N, None, None, 1, ws(nb), nb)
    assert within(rel_l2(host(C), C0 + A @ B), 1e-2)


def test_gemm_bias_gelu_and_dgelu():
    M, N, K = 520, 264, 392
    A, B, Ad, Bd = operands(3, M, N, K, 0, 1)
    bias = tp_synth.round_to_dtype(np.random.default_rng(4).standard_normal(N) * 0.3, "bf16")
    U, Y = empty((M, N), "bf16"), empty((M, N), "bf16")
    tp.tp_gemm_bf16(M, N, K, Ad, K, 0, Bd, N, 1, tp.TP_EPI_BIAS_GELU, U, Y, N, dev(bias, "bf16"), None, 0, None, 0)
    Uref = A @ B + bias
    assert within(rel_l2(host(U), Uref), 1e-2)
    assert within(rel_l2(host(Y), oracle.gelu(Uref)), 1e-2)
    # dGeLU: NT layout, aux = U as stored
    A2, B2, Ad2, Bd2 = operands(6, M, N, K, 0, 0)
    dU = empty((M, N), "bf16")
    tp.tp_gemm_bf16(M, N, K, Ad2, K, 0, Bd2, K, 0, tp.TP_EPI_DGELU, dU, None, N, None, U, 0, None, 0)
    assert within(rel_l2(host(dU), (A2 @ B2) * oracle.gelu_grad(host(U))), 1e-2)


def test_gemm_k_zero_and_refusals():
    M, N = 64, 64
    C = dev(np.full((M, N), 5.0), "bf16")
    dummy = empty((64,), "bf16")
    tp.tp_gemm_bf16(M, N, 0, dummy, 8, 0, dummy, 8, 0, tp.TP_EPI_STORE, C, None, N, None, None, 0, None, 0)
    assert np.all(host(C) == 0)
    with pytest.raises(tp.TPError):       # A MN-contiguous with B K-contiguous is not implemented
        tp.tp_gemm_bf16(M, N, 8, dummy, 64, 1, dummy, 8, 0, tp.TP_EPI_STORE, C, None, N, None, None, 0, None, 0)


def test_backward_calls_on_two_streams_are_independent():
    """Two MLP-shard backward calls with different inputs, issued on two streams at once, write
    exactly what the same calls write one after the other."""
    T, h, ffn, t = 1024, 512, 2048, 2
    Ft = ffn // t
    sets = []
    for seed in (11, 12):
        inp = tp_synth.mlp_inputs(seed, T, h, ffn, "bf16", bias_std=0.1)
        d = {k: dev(v, "bf16") for k, v in inp.items()}
        A_r, B_r, b1 = d["A"][:, :Ft].contiguous(), d["B"][:Ft].contiguous(), d["b1"][:Ft].contiguous()
        U, Y, Z = empty((T, Ft), "bf16"), empty((T, Ft), "bf16"), empty((T, h), "bf16")
        tp.tp_mlp_shard_fwd(T, h, ffn, t, 0, tp.TP_BF16, d["X"], A_r, b1, B_r, U, Y, Z)
        nb = tp.tp_mlp_shard_bwd_workspace(T, h, ffn, t, tp.TP_BF16)
        sets.append(dict(X=d["X"], G=d["G"], A=A_r, B=B_r, U=U, Y=Y, ws=ws(nb), nb=nb))
    torch.cuda.synchronize()

    def call(s, stream=None):
        outs = dict(dX=empty((T, h), "bf16"), dA=empty((h, Ft), "bf16"), db1=empty((Ft,), "bf16"),
                    dB=empty((Ft, h), "bf16"))
        tp.tp_mlp_shard_bwd(T, h, ffn, t, 0, tp.TP_BF16, s["X"], s["A"], s["B"], s["U"], s["Y"], s["G"], outs["dX"],
                            outs["dA"], outs["db1"], outs["dB"], 0, s["ws"], s["nb"], stream)
        return outs

    serial = [call(s) for s in sets]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    conc = [call(s, st.cuda_stream) for s, st in zip(sets, streams)]
    torch.cuda.synchronize()
    say("[streams] two backward calls at once")
    for a, b in zip(serial, conc):
        for k in a:
            assert torch.equal(a[k], b[k]), k
