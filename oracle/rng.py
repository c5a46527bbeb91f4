"""Counter-based random numbers and dropout masks: plain definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Passages: "Megatron-LM: Training Multi-Billion Parameter Language Models Using Model
Parallelism" (paper digest), §3.4, "Random Number Generation Handling": dropout inside the
attention block (a model-parallel region) must draw a different pattern on every rank, from a
generator seeded per rank; dropout on the residual connections, applied after g to data that is
identical on every rank, must draw the same pattern everywhere (one shared seed). "Megatron-LM,
annotated", §4.2: dropout probability 0.1.

Generator. The pages name none. A counter-based generator lets every element's draw be computed
on its own, in any order, on the GPU and here: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011). State: a counter of four 32-bit words
(c0, c1, c2, c3) and a key of two (k0, k1). One round maps the counter to
    (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))
with M0 = 0xD2511F53, M1 = 0xCD9E8D57 and hi/lo the upper/lower halves of the 64-bit product;
the key is bumped by (0x9E3779B9, 0xBB67AE85) before each of rounds 2..10.

Streams and element mapping (the library's own):
* key = (seed mod 2^32, seed div 2^32); c3 = stream; c2 = 0; (c0, c1) = the call index, a 64-bit
  number, low word in c0.
* one call gives eight 16-bit uniforms u[j] = (word j // 2 >> 16 (j % 2)) & 0xFFFF.
* keep an element iff u >= thr with thr = round(p 65536): p is quantised to a multiple of
  1/65536. Kept values are scaled by 65536 / (65536 - thr), the inverse of the exact keep
  probability, so dropout leaves the expectation unchanged.
* residual dropout over x [T, n]: element (t, c) is slot c % 8 of call t (n / 8) + c / 8.
* attention dropout over the probabilities P[q, k] of global head hg of sequence b (s queries per
  sequence, heads heads in all, n32 = ceil(s / 32) key tiles of 32): slot (k % 16) / 8 * 4 + k % 4
  of call ((((b heads + hg) s + q) n32 + k / 32) 2 + (k % 8) / 4) 2 + (k % 32) / 16. Per query
  and 32-key tile this groups the sixteen keys {8i + 4h + j} held by one GPU lane into two calls.
  The shared stream of the residual sites and the per-rank streams of the attention sites are
  chosen by the caller (the layer uses one stream id per residual site and one per rank).

Pins (``tests/test_oracle_rng.py``): rocRAND's own Philox4x32-10 (its header implementation,
compiled for the host) on many counters and keys; the attention mapping is a bijection onto
(call, slot) pairs; kept fractions and the unbiased scale within binomial bounds; streams and
seeds give independent patterns.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32", "uniform16", "drop_threshold", "drop_scale", "residual_keep",
           "attn_call_slot", "attn_keep", "dropout_apply"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on arrays of counter words (broadcast), scalar key; four uint32 arrays."""
    x = [np.asarray(c, dtype=np.uint64) & _LO for c in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for r in range(10):
        if r > 0:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * x[0]          # < 2^64: no wrap in uint64
        p1 = _M1 * x[2]
        x = [(p1 >> _SH) ^ x[1] ^ np.uint64(k0), p1 & _LO, (p0 >> _SH) ^ x[3] ^ np.uint64(k1), p0 & _LO]
    return [w.astype(np.uint32) for w in x]


def uniform16(call, seed: int, stream: int) -> np.ndarray:
    """The eight 16-bit uniforms of each call index (any integer array): shape call.shape + (8,)."""
    call = np.asarray(call, dtype=np.uint64)
    w = philox4x32(call & _LO, call >> _SH, 0, stream, seed & 0xFFFFFFFF, seed >> 32)
    out = np.empty(call.shape + (8,), dtype=np.uint16)
    for j in range(8):
        out[..., j] = (w[j // 2] >> np.uint32(16 * (j % 2))) & np.uint32(0xFFFF)
    return out


def drop_threshold(p: float) -> int:
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p * 65536.0 + 0.5))


def drop_scale(p: float) -> float:
    thr = drop_threshold(p)
    return 65536.0 / (65536 - thr)


def residual_keep(T: int, n: int, p: float, seed: int, stream: int) -> np.ndarray:
    """Keep mask [T, n] of a residual dropout site."""
    assert n % 8 == 0
    t = np.arange(T, dtype=np.uint64)[:, None]
    c = np.arange(n // 8, dtype=np.uint64)[None, :]
    u = uniform16(t * np.uint64(n // 8) + c, seed, stream)          # [T, n/8, 8]
    return u.reshape(T, n) >= drop_threshold(p)


def attn_call_slot(b, hg, q, k, heads: int, s: int):
    """(call index, slot) of attention element (sequence b, global head hg, query q, key k)."""
    b, hg, q, k = (np.asarray(v, dtype=np.int64) for v in (b, hg, q, k))
    n32 = (s + 31) // 32
    row = (b * heads + hg) * s + q
    call = (((row * n32 + k // 32) * 2 + (k % 8) // 4) * 2 + (k % 32) // 16)
    slot = ((k % 16) // 8) * 4 + k % 4
    return call, slot


def attn_keep(b: int, hg: int, s: int, heads: int, p: float, seed: int, stream: int,
              queries=None) -> np.ndarray:
    """Keep mask [len(queries), s] (keys 0..s-1) of head hg of sequence b (all queries by default)."""
    q = np.arange(s) if queries is None else np.asarray(queries)
    k = np.arange(s)
    call, slot = attn_call_slot(b, hg, q[:, None], k[None, :], heads, s)
    u = uniform16(call.astype(np.uint64), seed, stream)                    # [nq, s, 8]
    vals = np.take_along_axis(u, slot[..., None].astype(np.int64), axis=-1)[..., 0]
    return vals >= drop_threshold(p)


def dropout_apply(x: np.ndarray, keep: np.ndarray, p: float) -> np.ndarray:
    """x * keep * 65536 / (65536 - thr)."""
    return np.where(keep, x * drop_scale(p), 0.0)
