"""GPU parity of the fp8 (OCP E4M3) path through the C ABI against the float64 oracle
(oracle/fp8.py): per-tensor quantisation (codes, transposed codes, amax, descale: bit-exact) and
the fp8 GEMM with its epilogues.

GEMM tolerance: the oracle sums the same decoded codes in float64; the kernel accumulates exact
fp8 products in fp32 and rounds the result to bf16 (relative error <= 2^-9 per element), so the
relative L2 error is bounded near 2^-9 / sqrt(3) ~ 1.1e-3. The bar is 4e-3."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
import tp_synth
from tests.gpu_util import DEV, dev, empty, host, rel_l2, within, say, ws

pytestmark = pytest.mark.gpu
tp = pytest.importorskip("tensor_transformer_layer_amd")
TOL = 4e-3


def u8(shape):
    return torch.zeros(shape, dtype=torch.uint8, device=DEV)


def f32_scalar():
    return torch.full((4,), -1.0, dtype=torch.float32, device=DEV)   # 16-byte aligned, poisoned


def quantize(x, dtype, want_codes=True, want_t=True, pad=0):
    """Run tp_fp8_quantize on the float64 array x held in `dtype`; returns host copies."""
    rows, cols = x.shape
    X = dev(x, dtype)
    ldc = ((cols + 15) // 16) * 16 + pad
    ldt = ((rows + 15) // 16) * 16 + pad
    codes = u8((rows, ldc)) if want_codes else None
    codes_t = u8((cols, ldt)) if want_t else None
    amax, descale = f32_scalar(), f32_scalar()
    nb = tp.tp_fp8_quantize_workspace(rows, cols)
    tp.tp_fp8_quantize(rows, cols, tp.TP_BF16 if dtype == "bf16" else tp.TP_F32, X, cols, codes, ldc, codes_t,
                       ldt, amax, descale, ws(nb), nb)
    torch.cuda.synchronize()
    out = {"amax": float(amax[0].item()), "descale": float(descale[0].item())}
    if want_codes:
        out["codes"] = codes[:, :cols].cpu().numpy()
    if want_t:
        out["codes_t"] = codes_t[:, :rows].cpu().numpy()
    return out


def check_quant(x, dtype, got):
    codes, e, amax = f8.quantize(x)
    assert got["amax"] == amax
    assert got["descale"] == math.ldexp(1.0, -e)
    if "codes" in got:
        bad = np.argwhere(got["codes"] != codes)
        assert bad.size == 0, (bad[:5], got["codes"][tuple(bad[0])], codes[tuple(bad[0])])
    if "codes_t" in got:
        assert np.array_equal(got["codes_t"], codes.T)
    return e


def all_bf16_in_range():
    """Every bf16 value with magnitude <= 448, as float64 (31,618 values incl. +-0)."""
    u = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    v = u.view(np.float32)
    v = v[np.isfinite(v)].astype(np.float64)
    return v[np.abs(v) <= 448]


@pytest.mark.parametrize("shift", [0, 5, -7])
def test_fp8_quantize_every_bf16_value(shift):
    """All bf16 values in [-448, 448] times 2^-shift (exact in bf16), one tensor: amax = 448 * 2^-shift,
    so e = shift and every value's code is the conversion of the value itself."""
    v = all_bf16_in_range() * math.ldexp(1.0, -shift)
    n = (len(v) + 127) // 128 * 128
    x = np.zeros(n)
    x[:len(v)] = v
    x = x.reshape(-1, 128)
    say(f"[fp8] quantize all bf16 values, shift={shift}, shape={x.shape}")
    got = quantize(x, "bf16")
    assert check_quant(x, "bf16", got) == shift


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1000, 136), (67, 8), (64, 128), (129, 3072)])
def test_fp8_quantize_ragged(dtype, rows, cols):
    x = tp_synth.normal(600 + rows, 1, (rows, cols), 0.02, dtype)
    x[rows // 2, cols // 3] = 0.5    # amax set by one element
    say(f"[fp8] quantize {dtype} {rows}x{cols}")
    check_quant(x, dtype, quantize(x, dtype, pad=16))


def test_fp8_quantize_degenerate():
    say("[fp8] quantize degenerate cases")
    # all zeros: e = 0, descale 1
    x = np.zeros((40, 24))
    got = quantize(x, "bf16")
    assert got["descale"] == 1.0 and got["amax"] == 0.0 and not got["codes"].any()
    # a tiny amax (bf16 subnormal): e clamps at 126
    x = np.zeros((16, 16))
    x[3, 5] = 2.0 ** -130
    x[7, 9] = -(2.0 ** -131)
    got = quantize(x, "bf16")
    assert check_quant(x, "bf16", got) == 126
    # one codes layout only
    x = tp_synth.normal(611, 1, (48, 64), 1.0, "bf16")
    check_quant(x, "bf16", quantize(x, "bf16", want_t=False))
    check_quant(x, "bf16", quantize(x, "bf16", want_codes=False))
    # zero rows still writes descale = 1 and amax = 0
    amax, descale = f32_scalar(), f32_scalar()
    nb = tp.tp_fp8_quantize_workspace(0, 64)
    tp.tp_fp8_quantize(0, 64, tp.TP_BF16, empty((1, 64), "bf16"), 64, u8((1, 64)), 64, None, 16, amax, descale,
                       ws(nb), nb)
    torch.cuda.synchronize()
    assert descale[0].item() == 1.0 and amax[0].item() == 0.0


def run_gemm(ca, da, cb, db, M, N, K, epi, bias=None, aux=None, C0=None, accumulate=0, use_ws=True, ldc=None):
    ldc = ldc or N
    lda = max(16, ((K + 15) // 16) * 16)
    A = u8((max(M, 1), lda)); A[:M, :K] = torch.from_numpy(ca).to(DEV)
    B = u8((max(N, 1), lda)); B[:N, :K] = torch.from_numpy(cb).to(DEV)
    sa = torch.tensor([math.ldexp(1.0, -da)] * 4, dtype=torch.float32, device=DEV)
    sb = torch.tensor([math.ldexp(1.0, -db)] * 4, dtype=torch.float32, device=DEV)
    Cm = dev(C0, "bf16") if C0 is not None else empty((max(M, 1), ldc), "bf16")
    C2 = empty((max(M, 1), ldc), "bf16") if epi == tp.TP_EPI_BIAS_GELU else None
    nb = tp.tp_gemm_fp8_workspace(M, N, K) if use_ws else 0
    tp.tp_gemm_fp8(M, N, K, A, lda, sa, B, lda, sb, epi, Cm, C2, ldc,
                   dev(bias, "bf16") if bias is not None else None, dev(aux, "bf16") if aux is not None else None,
                   accumulate, ws(nb) if nb else None, nb)
    out = host(Cm)[:M, :N]
    return (out, host(C2)[:M, :N]) if C2 is not None else out


def codes_of(seed, rows, cols, std):
    x = tp_synth.normal(seed, 1, (rows, cols), std, "bf16")
    c, e, _ = f8.quantize(x)
    return c, e


@pytest.mark.parametrize("M,N,K", [(300, 136, 272), (512, 384, 1024), (257, 200, 16), (64, 64, 4096)])
def test_gemm_fp8_store(M, N, K):
    ca, da = codes_of(700 + M, M, K, 1.0)
    cb, db = codes_of(800 + N, N, K, 0.02)
    ref = f8.gemm_fp8(ca, da, cb, db)
    say(f"[fp8] gemm store M={M} N={N} K={K}")
    got = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_STORE)
    e = rel_l2(got, ref)
    say(f"  rel_l2={e:.2e}")
    assert within(e, TOL)
    # bias + accumulate into a padded output
    bias = tp_synth.normal(901, 1, (N,), 0.5, "bf16")
    C0 = np.zeros((M, N + 8))
    C0[:, :N] = tp_synth.normal(902, 1, (M, N), 0.5, "bf16")
    got = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_STORE, bias=bias, C0=C0, accumulate=1, ldc=N + 8)
    e = rel_l2(got, ref + bias[None, :] + C0[:, :N])
    say(f"  bias+accumulate rel_l2={e:.2e}")
    assert within(e, TOL)


def test_gemm_fp8_epilogues():
    M, N, K = 333, 264, 512
    ca, da = codes_of(710, M, K, 1.0)
    cb, db = codes_of(810, N, K, 0.05)
    P = f8.gemm_fp8(ca, da, cb, db)
    bias = tp_synth.normal(911, 1, (N,), 0.5, "bf16")
    say("[fp8] gemm bias+gelu")
    U, Y = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_BIAS_GELU, bias=bias)
    Uref = P + bias[None, :]
    assert within(rel_l2(U, Uref), TOL)
    assert within(rel_l2(Y, oracle.gelu(Uref)), TOL)
    say("[fp8] gemm dgelu")
    aux = tp_synth.normal(912, 1, (M, N), 1.0, "bf16")
    dU = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_DGELU, aux=aux)
    assert within(rel_l2(dU, P * oracle.gelu_grad(aux)), TOL)


def test_gemm_fp8_split_k_matches_unsplit_and_is_deterministic():
    """A weight-gradient shape (long K): with the workspace the plan may split K; the result is the
    same GEMM and repeated calls give identical bits."""
    M, N, K = 384, 512, 8192
    ca, da = codes_of(720, M, K, 1.0)
    cb, db = codes_of(820, N, K, 1.0)
    ref = f8.gemm_fp8(ca, da, cb, db)
    say(f"[fp8] gemm split-K M={M} N={N} K={K} ws={tp.tp_gemm_fp8_workspace(M, N, K)}")
    a = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_STORE, use_ws=True)
    b = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_STORE, use_ws=True)
    c = run_gemm(ca, da, cb, db, M, N, K, tp.TP_EPI_STORE, use_ws=False)
    assert np.array_equal(a, b)
    assert within(rel_l2(a, ref) <= TOL and rel_l2(c, ref), TOL)


def test_gemm_fp8_zero_k_and_empty():
    say("[fp8] gemm K=0 and M=0")
    M, N = 70, 24
    bias = tp_synth.normal(921, 1, (N,), 0.5, "bf16")
    out = run_gemm(np.zeros((M, 0), np.uint8), 0, np.zeros((N, 0), np.uint8), 0, M, N, 0, tp.TP_EPI_STORE,
                   bias=bias, use_ws=False)
    assert np.array_equal(out, np.broadcast_to(bias, (M, N)))
    run_gemm(np.zeros((0, 32), np.uint8), 0, np.zeros((N, 32), np.uint8), 0, 0, N, 32, tp.TP_EPI_STORE)


# the fp8 GEMMs of one rank of the 8.3B-shape layer (t = 8, 8192 tokens, h = 3072, ffn/t = 1536)
LAYER_SHAPES = [
    ("mlp1_fwd", 8192, 1536, 3072, "bias_gelu"),
    ("mlp2_fwd", 8192, 3072, 1536, "store"),
    ("dB_wgrad", 1536, 3072, 8192, "store"),
]


@pytest.mark.parametrize("name,M,N,K,epi", LAYER_SHAPES)
def test_gemm_fp8_full_size_sampled(name, M, N, K, epi):
    """Full-size layer GEMMs, quantised on the GPU from bf16 inputs; the codes are checked
    bit-exact on sampled rows and the products on 64 sampled rows of the output."""
    g = np.random.default_rng(930)
    xa = tp_synth.normal(931, 1, (M, K), 1.0, "bf16")
    xb = tp_synth.normal(932, 1, (N, K), 0.02, "bf16")
    say(f"[fp8] full-size {name} M={M} N={N} K={K} {epi}")
    qa = quantize(xa, "bf16", want_t=False)
    qb = quantize(xb, "bf16", want_t=False)
    rows = np.sort(g.choice(M, 64, replace=False))
    ea = f8.scale_exponent(np.max(np.abs(xa)))
    eb = f8.scale_exponent(np.max(np.abs(xb)))
    assert qa["descale"] == math.ldexp(1.0, -ea) and qb["descale"] == math.ldexp(1.0, -eb)
    assert np.array_equal(qa["codes"][rows], f8.e4m3_encode(xa[rows] * math.ldexp(1.0, ea)))
    assert np.array_equal(qb["codes"][::97], f8.e4m3_encode(xb[::97] * math.ldexp(1.0, eb)))
    kind = tp.TP_EPI_BIAS_GELU if epi == "bias_gelu" else tp.TP_EPI_STORE
    bias = tp_synth.normal(933, 1, (N,), 0.5, "bf16") if epi == "bias_gelu" else None
    out = run_gemm(qa["codes"], ea, qb["codes"], eb, M, N, K, kind, bias=bias)
    if kind == tp.TP_EPI_BIAS_GELU:
        out = out[1]
    ref = f8.gemm_fp8(qa["codes"][rows], ea, qb["codes"], eb)
    if kind == tp.TP_EPI_BIAS_GELU:
        ref = oracle.gelu(ref + bias[None, :])
    e = rel_l2(out[rows], ref)
    say(f"  sampled rel_l2={e:.2e}")
    assert within(e, TOL)
