"""Pins for the vocabulary-parallel embedding oracle (oracle/embedding.py)."""
import numpy as np
import torch

import oracle.embedding as emb


def _case(seed=3, N=97, V=64, h=24):
    g = np.random.default_rng(seed)
    ids = g.integers(0, V, N)
    ids[:4] = [0, V - 1, V // 4 - 1, V // 4]     # shard boundaries for t = 4
    ids[10:20] = 7                                # a repeated id
    return ids, g.standard_normal((V, h)), g.standard_normal((N, h))


def test_partials_sum_to_lookup_and_match_torch():
    ids, E, _ = _case()
    V, t = E.shape[0], 4
    Vt = V // t
    parts = [emb.embed_shard_fwd(ids, E[r * Vt:(r + 1) * Vt], r) for r in range(t)]
    want = torch.nn.functional.embedding(torch.from_numpy(ids), torch.from_numpy(E)).numpy()
    assert np.array_equal(sum(parts), want)
    assert np.array_equal(emb.embed_full(ids, E), want)
    # each token is non-zero on exactly one rank
    nz = np.stack([np.any(p != 0, axis=1) for p in parts])
    assert np.array_equal(nz.sum(axis=0), np.ones(len(ids)))


def test_backward_matches_autograd_and_split():
    ids, E, G = _case()
    V, t = E.shape[0], 4
    Vt = V // t
    Et = torch.from_numpy(E).requires_grad_(True)
    torch.nn.functional.embedding(torch.from_numpy(ids), Et).backward(torch.from_numpy(G))
    full = emb.embed_full_bwd(ids, G, V)
    assert np.allclose(full, Et.grad.numpy(), rtol=0, atol=1e-12)
    for r in range(t):
        assert np.array_equal(emb.embed_shard_bwd(ids, G, Vt, r), full[r * Vt:(r + 1) * Vt])


def test_out_of_shard_ids_give_zero_rows():
    E_r = np.ones((8, 4))
    out = emb.embed_shard_fwd(np.array([7, 8, 15, 16, 0]), E_r, 1)   # rank 1 owns ids 8..15
    assert np.array_equal(out.any(axis=1), [False, True, True, False, False])
