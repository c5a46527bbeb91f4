"""Vocabulary-parallel input embedding, forward and backward, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Passage: "Megatron-LM: Training Multi-Billion Parameter Language Models Using Model
Parallelism" (paper digest), §3.4, "Input Embedding Parallelism": the table E [V, h] is split
over vocabulary entries into t row blocks E_r [V/t, h]; rank r looks up the tokens whose ids fall
in its block and returns a zero row for every other token; g (all-reduce) sums the ranks'
partials, which rebuilds E[ids] on every rank since each id lives on exactly one rank.
(The pages call the split "column-wise along the vocabulary dimension" while writing row blocks
E_i of shape [vocabulary/n, hidden]; both describe a split over vocabulary entries.)

Backward (not on the pages; the derivative of a lookup): with G = dL/d(embedded tokens) [N, h],
replicated after g, dE[v] = sum of G[i] over the tokens i with ids[i] = v; rank r owns rows
r V_t .. (r + 1) V_t - 1 of it.

Pins (``tests/test_oracle_embedding.py``): the ranks' partials sum to the unsplit lookup;
PyTorch CPU float64 ``nn.functional.embedding`` and its autograd backward; the shard backward
equals the owned rows of the unsplit backward; out-of-shard and boundary ids.
"""
from __future__ import annotations

import numpy as np

__all__ = ["embed_full", "embed_shard_fwd", "embed_full_bwd", "embed_shard_bwd"]


def embed_full(ids: np.ndarray, E: np.ndarray) -> np.ndarray:
    """E[ids]: [N, h]."""
    return E[np.asarray(ids)]


def embed_shard_fwd(ids: np.ndarray, E_r: np.ndarray, r: int) -> np.ndarray:
    """Rank r's partial: E_r[ids - r V_t] for ids in [r V_t, (r + 1) V_t), else a zero row."""
    Vt, h = E_r.shape
    ids = np.asarray(ids, dtype=np.int64)
    local = ids - r * Vt
    own = (local >= 0) & (local < Vt)
    out = np.zeros((ids.size, h))
    out[own] = E_r[local[own]]
    return out


def embed_full_bwd(ids: np.ndarray, G: np.ndarray, V: int) -> np.ndarray:
    """dE [V, h]: row v is the sum of G[i] over the tokens with ids[i] = v (tokens in order)."""
    dE = np.zeros((V, G.shape[1]))
    for i, v in enumerate(np.asarray(ids)):
        dE[v] += G[i]
    return dE


def embed_shard_bwd(ids: np.ndarray, G: np.ndarray, Vt: int, r: int) -> np.ndarray:
    """Rank r's rows of dE: [V_t, h]."""
    dE = np.zeros((Vt, G.shape[1]))
    for i, v in enumerate(np.asarray(ids, dtype=np.int64)):
        if r * Vt <= v < (r + 1) * Vt:
            dE[v - r * Vt] += G[i]
    return dE
