"""Pins for the fp8 oracle (oracle/fp8.py): the E4M3 format, the per-tensor power-of-two scale
and the fp8 GEMM, each checked against something other than the oracle itself."""
import math

import numpy as np
import pytest
import torch

import oracle.fp8 as f8


def test_e4m3_closed_form_codes():
    # values fixed by the format's fields: sign | exponent (bias 7) | mantissa
    cases = {
        1.0: 0x38,            # E = 7, m = 0
        448.0: 0x7E,          # E = 15, m = 6: the largest finite magnitude
        -2.0: 0xC0,           # sign, E = 8
        2.0 ** -9: 0x01,      # smallest subnormal, 1/8 * 2^-6
        7 * 2.0 ** -9: 0x07,  # largest subnormal
        2.0 ** -6: 0x08,      # smallest normal
        1.875: 0x3F,          # (1 + 7/8) * 2^0
        0.0: 0x00,
    }
    for v, code in cases.items():
        assert f8.e4m3_encode(np.array([v]))[0] == code, v
        assert f8.e4m3_decode(np.array([code], dtype=np.uint8))[0] == v
    assert f8.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert math.isnan(f8.e4m3_decode(np.array([0x7F], dtype=np.uint8))[0])
    assert math.isnan(f8.e4m3_decode(np.array([0xFF], dtype=np.uint8))[0])
    assert f8.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_e4m3_table_shape_of_the_format():
    t = f8.e4m3_decode_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # monotone in the code
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])       # sign bit only flips the sign
    # spacing: 2^-9 through the subnormals and first binade, then doubling per binade
    assert np.allclose(np.diff(pos[:16]), 2.0 ** -9)
    for e in range(1, 15):
        binade = pos[8 * e: 8 * e + 8]
        assert np.allclose(np.diff(binade), 2.0 ** (e - 7) / 8)


def test_e4m3_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(f8.e4m3_encode(f8.e4m3_decode(codes)), codes)


def test_e4m3_ties_to_even_and_neighbours():
    t = f8.e4m3_decode_table()
    for c in range(0, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert f8.e4m3_encode(np.array([mid]))[0] == even
        assert f8.e4m3_encode(np.array([np.nextafter(mid, -np.inf)]))[0] == c
        assert f8.e4m3_encode(np.array([np.nextafter(mid, np.inf)]))[0] == c + 1
        assert f8.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)


def test_e4m3_saturates():
    for v in (448.0, 449.0, 464.0, 1e6, np.finfo(np.float64).max):
        assert f8.e4m3_encode(np.array([v]))[0] == 0x7E
        assert f8.e4m3_encode(np.array([-v]))[0] == 0xFE


def test_e4m3_matches_torch_on_every_bf16_in_range():
    # PyTorch's float8_e4m3fn cast (round to nearest even) over all 65,536 bf16 patterns whose
    # magnitude is at most 448; outside that range PyTorch gives NaN where this scheme saturates.
    b = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()
    b = b[torch.isfinite(b) & (b.abs() <= 448)]
    want = b.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = f8.e4m3_encode(b.double().numpy())
    assert np.array_equal(got, want)
    # and on random fp32 values spread over the whole range, subnormals included
    g = np.random.default_rng(7)
    x = (g.standard_normal(200_000) * np.exp2(g.uniform(-12, 8.7, 200_000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f8.e4m3_encode(x.astype(np.float64)), want)


@pytest.mark.parametrize("amax,e", [(1.0, 8), (448.0, 0), (449.0, -1), (3.5, 7), (3.5000001, 6),
                                    (224.0, 1), (224.00001, 0), (2.0 ** -20, 28), (0.0, 0)])
def test_scale_exponent_closed_form(amax, e):
    assert f8.scale_exponent(amax) == e


def test_scale_exponent_defining_inequality():
    g = np.random.default_rng(11)
    for amax in np.exp2(g.uniform(-60, 60, 2000)):
        e = f8.scale_exponent(amax)
        # exact rational check with Python's arbitrary-precision integers via fractions
        from fractions import Fraction
        s = Fraction(amax) * (Fraction(2) ** e)
        assert s <= 448 < 2 * s
    assert f8.scale_exponent(1e-300) == 126     # clamped
    assert f8.scale_exponent(1e300) == -126     # clamped


def test_quantize_scaled_range_and_dequant_error():
    g = np.random.default_rng(3)
    x = g.standard_normal((64, 96)) * 0.02
    codes, e, amax = f8.quantize(x)
    assert amax == np.max(np.abs(x))
    y = f8.e4m3_decode(codes) * 2.0 ** -e
    # the largest element lands in (224, 448]; relative error of normal values is <= 2^-4
    assert 224 < amax * 2.0 ** e <= 448
    big = np.abs(x) * 2.0 ** e >= 2.0 ** -6
    assert np.all(np.abs(y[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4)
    assert np.all(np.abs(y[~big] - x[~big]) <= 2.0 ** -10 * 2.0 ** -e)


def test_gemm_fp8_integer_brute_force():
    # integers of magnitude <= 16 are exact in E4M3 (3 mantissa bits), so after the power-of-two
    # scale the GEMM must equal the integer product exactly
    g = np.random.default_rng(5)
    M, N, K = 5, 4, 7
    a = g.integers(-8, 9, size=(M, K)).astype(np.float64)
    b = g.integers(-8, 9, size=(N, K)).astype(np.float64)
    a[0, 0], b[0, 0] = 8.0, -8.0
    ca, ea, _ = f8.quantize(a)
    cb, eb, _ = f8.quantize(b)
    assert ea == 5 and eb == 5          # 8 * 2^5 = 256 <= 448 < 512
    c = f8.gemm_fp8(ca, ea, cb, eb)
    for m in range(M):
        for n in range(N):
            ref = 0
            for k in range(K):
                ref += int(a[m, k]) * int(b[n, k])
            assert c[m, n] == ref


def test_gemm_fp8_scaling_is_exact():
    # multiplying an input by a power of two shifts its exponent and leaves the codes alone
    g = np.random.default_rng(9)
    a = g.standard_normal((8, 32))
    b = g.standard_normal((6, 32))
    ca, ea, _ = f8.quantize(a)
    cb, eb, _ = f8.quantize(b)
    ca2, ea2, _ = f8.quantize(a * 64.0)
    assert np.array_equal(ca, ca2) and ea2 == ea - 6
    assert np.array_equal(f8.gemm_fp8(ca2, ea2, cb, eb), f8.gemm_fp8(ca, ea, cb, eb) * 64.0)
