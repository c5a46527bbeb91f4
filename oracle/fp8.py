"""fp8 (OCP E4M3) quantisation and the fp8 GEMM: plain fp64 CPU definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke check
and the bench's CPU baseline, never by the GPU library.

Context. The pages train in 16-bit floating point with dynamic loss scaling ("Megatron-LM,
annotated", §4.2 Training optimization and hyperparameters; the Chinese reading notes on the
same paper, section on mixed precision and memory management) and define no 8-bit format.
Everything below is therefore the library's own scheme, written out as definitions:

* Format: E4M3 of the OCP 8-bit floating-point specification. Bit 7 is the sign, bits 6..3 the
  exponent field E (bias 7), bits 2..0 the mantissa field m. E = 0 encodes the subnormals
  m/8 * 2^-6; E = 1..15 encodes (1 + m/8) * 2^(E-7), except E = 15, m = 7, which is NaN. There
  are no infinities; the largest finite magnitude is 448 (E = 15, m = 6).
* Conversion of a real x: the nearest finite E4M3 value, ties to the code whose mantissa field
  is even; magnitudes above 448 saturate to 448; the sign is kept (so -0 and tiny negatives give
  code 0x80); NaN gives 0x7F.
* Per-tensor scaling: amax = max |x| over the tensor; the scale is 2^e with e the largest
  integer such that amax * 2^e <= 448 (e = 0 when amax = 0 or is not finite), clamped to
  [-126, 126] so that 2^e and 2^-e are both normal fp32 numbers. A power of two makes x * 2^e
  exact, so the only rounding is the conversion itself, and 2^-e undoes the scale exactly.
* GEMM: C[m, n] = 2^-(e_a + e_b) * sum_k dec(a[m, k]) * dec(b[n, k]) in fp64, with both code
  matrices K-contiguous (a is [M, K], b is [N, K]).

Pins (``tests/test_oracle_fp8.py``): closed-form codes of the format (1, 448, the smallest
subnormal and normal, -2), the decode/encode round trip over all finite codes, ties to even at
midpoints, saturation, PyTorch's own float8_e4m3fn conversion over every bf16 value in
[-448, 448] (an independent library routine), the scale exponent's defining inequality on
random and boundary amax values, and the GEMM against an integer brute-force product on
integer-valued inputs that the format holds exactly.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_decode_table", "e4m3_decode", "e4m3_encode", "scale_exponent",
           "quantize", "gemm_fp8"]

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (float64; NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 15 and m == 7:
            vals[code] = math.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
# non-negative finite codes 0x00..0x7E in increasing value order (the encoding is monotone)
_POS_VALS = _TABLE[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round real values (any float array) to E4M3 codes (uint8), as defined in the header."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_x)
    neg = np.signbit(flat_x)
    a = np.minimum(np.abs(np.where(nan, 0.0, flat_x)), E4M3_MAX)
    # the two finite neighbours lo <= a <= hi
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.where(_POS_VALS[hi] == a, hi, np.maximum(hi - 1, 0))
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(neg, code | np.uint8(0x80), code)
    flat_o[:] = np.where(nan, np.uint8(0x7F), code)
    return out


def scale_exponent(amax: float) -> int:
    """Largest integer e with amax * 2^e <= 448, clamped to [-126, 126]; 0 for amax = 0.

    Found by the defining inequality itself: a first guess from log2, then moved by whole
    steps until amax * 2^e <= 448 < amax * 2^(e+1) holds (products by powers of two are exact
    in float64 over this range).
    """
    amax = float(amax)
    if amax == 0.0 or not math.isfinite(amax):
        return 0
    e = int(math.floor(math.log2(E4M3_MAX / amax)))
    while math.ldexp(amax, e) > E4M3_MAX:
        e -= 1
    while math.ldexp(amax, e + 1) <= E4M3_MAX:
        e += 1
    return max(-126, min(126, e))


def quantize(x: np.ndarray):
    """Per-tensor fp8 quantisation of x (float values, e.g. bf16 held in float64).

    Returns (codes uint8 of x's shape, e, amax). Dequantised values are dec(codes) * 2^-e.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    e = scale_exponent(amax)
    codes = e4m3_encode(x * math.ldexp(1.0, e))
    return codes, e, amax


def gemm_fp8(a_codes: np.ndarray, e_a: int, b_codes: np.ndarray, e_b: int) -> np.ndarray:
    """C[M, N] = 2^-(e_a + e_b) * dec(a)[M, K] @ dec(b)[N, K]^T, float64."""
    a = e4m3_decode(a_codes)
    b = e4m3_decode(b_codes)
    return (a @ b.T) * math.ldexp(1.0, -(e_a + e_b))
