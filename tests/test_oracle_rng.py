"""Pins for the counter-based generator and the dropout masks (oracle/rng.py)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle.rng as rng

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    """rocRAND's Philox4x32-10, built from its header for the host (no GPU involved)."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "ref")
    r = subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"),
                        "-o", exe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        pytest.skip("could not build the rocRAND reference: " + r.stderr[-500:])

    def run(seed, sub, off, n):
        out = subprocess.run([exe, hex(seed), hex(sub), hex(off), str(n)], capture_output=True, text=True,
                             check=True).stdout.split()
        return np.array([int(w, 16) for w in out], dtype=np.uint64).reshape(n, 4)
    return run


@pytest.mark.parametrize("seed,sub,off", [(0, 0, 0), (0x0123456789ABCDEF, 5, 8), (2**64 - 1, 2**63 + 7, 4 * 12345),
                                          (42, 0, 4 * (2**32 - 2)), (7, 2**40 + 3, 4 * (2**33 + 1))])
def test_philox_matches_rocrand(rocrand_ref, seed, sub, off):
    n = 6
    want = rocrand_ref(seed, sub, off, n)
    ctr = off // 4 + np.arange(n, dtype=np.uint64)
    got = rng.philox4x32(ctr & 0xFFFFFFFF, ctr >> 32, sub & 0xFFFFFFFF, sub >> 32, seed & 0xFFFFFFFF, seed >> 32)
    got = np.stack([g.astype(np.uint64) for g in got], axis=1)
    assert np.array_equal(got, want)


def test_uniform16_unpacks_words_low_half_first():
    call = np.array([0, 1, 2**33 + 5], dtype=np.uint64)
    u = rng.uniform16(call, 99, 3)
    w = rng.philox4x32(call & 0xFFFFFFFF, call >> 32, 0, 3, 99, 0)
    for j in range(8):
        assert np.array_equal(u[:, j], (w[j // 2] >> (16 * (j % 2))) & 0xFFFF)


def test_threshold_and_scale():
    assert rng.drop_threshold(0.0) == 0 and rng.drop_scale(0.0) == 1.0
    assert rng.drop_threshold(0.1) == 6554
    assert rng.drop_scale(0.5) == 2.0
    with pytest.raises(ValueError):
        rng.drop_threshold(1.0)


def test_attention_mapping_is_a_bijection():
    b, heads, s = 2, 3, 80            # s not a multiple of 32: the last key tile is ragged
    B, H, Q, K = np.meshgrid(np.arange(b), np.arange(heads), np.arange(s), np.arange(s), indexing="ij")
    call, slot = rng.attn_call_slot(B, H, Q, K, heads, s)
    key = call * 8 + slot
    assert len(np.unique(key)) == key.size
    # one lane's sixteen keys (query q, tile kt, half h) are exactly two whole calls
    q, kt, h = 17, 1, 1
    ks = np.array([32 * kt + 8 * (v // 4) + 4 * h + v % 4 for v in range(16)])
    c, sl = rng.attn_call_slot(1, 2, q, ks, heads, s)
    assert np.array_equal(sl, np.arange(16) % 8)
    assert np.array_equal(c, c[0] + np.arange(16) // 8)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_keep_fraction_and_unbiased_scale(p):
    keep = rng.residual_keep(512, 256, p, seed=1234, stream=0)
    n = keep.size
    q = 1 - rng.drop_threshold(p) / 65536
    assert abs(keep.mean() - q) < 5 * np.sqrt(q * (1 - q) / n)
    x = np.ones((512, 256))
    assert abs(rng.dropout_apply(x, keep, p).mean() - 1.0) < 5 * np.sqrt((1 - q) / (q * n))
    ka = rng.attn_keep(1, 2, 300, 4, p, seed=77, stream=9)
    assert abs(ka.mean() - q) < 5 * np.sqrt(q * (1 - q) / ka.size)


def test_streams_and_seeds_are_independent():
    a = rng.residual_keep(64, 512, 0.5, seed=5, stream=0)
    b = rng.residual_keep(64, 512, 0.5, seed=5, stream=1)
    c = rng.residual_keep(64, 512, 0.5, seed=6, stream=0)
    assert np.array_equal(a, rng.residual_keep(64, 512, 0.5, seed=5, stream=0))
    for o in (b, c):
        agree = (a == o).mean()
        assert 0.45 < agree < 0.55
    # the attention mask of the same head under two ranks' streams
    r0 = rng.attn_keep(0, 1, 128, 8, 0.5, seed=5, stream=100)
    r1 = rng.attn_keep(0, 1, 128, 8, 0.5, seed=5, stream=101)
    assert 0.45 < (r0 == r1).mean() < 0.55


def test_attn_keep_rows_subset():
    full = rng.attn_keep(1, 3, 100, 4, 0.2, seed=8, stream=4)
    rows = np.array([0, 31, 32, 99])
    assert np.array_equal(rng.attn_keep(1, 3, 100, 4, 0.2, seed=8, stream=4, queries=rows), full[rows])
