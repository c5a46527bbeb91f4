"""Vocabulary-parallel logits + cross-entropy, float64.

Test infrastructure only (see the package header).

Passages: "Megatron-LM: Training ... Model Parallelism" (paper digest), §3.4 "Output
Embedding Parallelism and the Fused Cross-Entropy Optimization" (logits Y_i = X E_i^T on the
rank's vocabulary rows; per-rank max, global max, per-rank sums of shifted exponentials,
global sum, loss from log s and the correct logit; weight tying; padding the vocabulary so
each rank's share is a multiple of 128) and "Megatron-LM, annotated", §3.4 The embedding
and the loss (51,200 = ceil(50,257 / 1,024) * 1,024; 943 padding rows; b*s numbers are
exchanged, not b*s*v).

Readings where the pages are silent or garbled:
* the max is per token (a row max over the rank's vocabulary);
* the printed loss "log(s) minus the correct logit" drops the max shift; with s taken
  relative to the global max M the loss is M + log s - y_target;
* the one-round merge (each rank keeps its own max; sums are rescaled when merged) equals
  the pages' two-round scheme in exact arithmetic; both are coded;
* padding columns are ordinary logits unless ``mask_padding`` (then they are -inf);
* rank r owns global columns [r*V_t, (r+1)*V_t); a rank that does not own the target
  reports 0 for it; argmax ties go to the lowest global index.

Pins: the padding arithmetic of "Megatron-LM, annotated" §3.4 (tests/golden); PyTorch CPU
float64 cross_entropy for the unsplit loss; one-round == two-round == unsplit; argmax and max
against numpy on the full logits. Backward: PyTorch CPU float64 autograd of the weighted
cross-entropy (with and without the padding mask); central finite differences of the forward
loss on every input entry; the rank split (sum of dX_r, stacked dE_r) against the unsplit
gradients; per-token logits gradients summing to zero; the uniform-logits closed form.
"""
import numpy as np


def pad_vocab(v, t, multiple=128):
    """Smallest multiple of multiple*t that is >= v."""
    q = multiple * t
    return -(-v // q) * q


def vocab_shard(E, t, r):
    """Rank r's rows of the tied embedding: [r*V/t, (r+1)*V/t)."""
    V = E.shape[0]
    assert V % t == 0
    w = V // t
    return E[r * w:(r + 1) * w]


def _masked_logits(X, E_rows, col0, Vreal, mask_padding):
    y = X @ E_rows.T
    if mask_padding:
        cols = col0 + np.arange(E_rows.shape[0])
        y = np.where(cols[None, :] < Vreal, y, -np.inf)
    return y


def xent_full(X, E, targets, Vreal, mask_padding=False):
    """Unsplit: loss_n = logsumexp_v(y_n) - y_n[target_n], y = X E^T."""
    y = _masked_logits(X, E, 0, Vreal, mask_padding)
    m = y.max(axis=1)
    lse = m + np.log(np.exp(y - m[:, None]).sum(axis=1))
    n = np.arange(X.shape[0])
    return {"loss": lse - y[n, targets], "max": m, "argmax": y.argmax(axis=1), "logits": y}


def xent_shard_stats(X, E_r, targets, t, r, Vreal, mask_padding=False):
    """One rank's per-token statistics: own max, sum of exp relative to it, the target's
    logit if this rank owns it (else 0), and the argmax as a global column index."""
    Vt = E_r.shape[0]
    col0 = r * Vt
    y = _masked_logits(X, E_r, col0, Vreal, mask_padding)
    m = y.max(axis=1)
    with np.errstate(invalid="ignore"):
        s = np.where(np.isfinite(m), np.exp(y - m[:, None]).sum(axis=1), 0.0)
    local = targets.astype(np.int64) - col0
    owned = (local >= 0) & (local < Vt)
    n = np.arange(X.shape[0])
    tgt = np.where(owned, y[n, np.clip(local, 0, Vt - 1)], 0.0)
    return {"max": m, "sumexp": s, "tgt": tgt, "argmax": y.argmax(axis=1) + col0, "logits": y}


def xent_combine(maxes, sumexps, tgts):
    """One-round merge of t ranks' statistics into per-token losses."""
    Mx = np.max(np.stack(maxes), axis=0)
    S = sum(s * np.exp(m - Mx) for m, s in zip(maxes, sumexps))
    return Mx + np.log(S) - sum(tgts)


def xent_two_round(X, E, targets, t, Vreal, mask_padding=False):
    """The pages' scheme: round 1 all-reduces the per-rank maxima to M; round 2 all-reduces
    each rank's sum of exp(y - M) and the owned target logits; loss = M + log s - y_target."""
    shards = [vocab_shard(E, t, r) for r in range(t)]
    Vt = shards[0].shape[0]
    ys = [_masked_logits(X, Er, r * Vt, Vreal, mask_padding) for r, Er in enumerate(shards)]
    Mx = np.max(np.stack([y.max(axis=1) for y in ys]), axis=0)
    s = sum(np.exp(y - Mx[:, None]).sum(axis=1) for y in ys)
    n = np.arange(X.shape[0])
    tgt = np.zeros(X.shape[0])
    for r, y in enumerate(ys):
        local = targets.astype(np.int64) - r * Vt
        owned = (local >= 0) & (local < Vt)
        tgt += np.where(owned, y[n, np.clip(local, 0, Vt - 1)], 0.0)
    return Mx + np.log(s) - tgt


# ------------------------------------------------------------------------------------------
# Backward. The pages give only the forward; the gradient is the textbook derivative of the
# same loss: d loss_n / d y_{n,v} = softmax_v(y_n) - [v == target_n]. Readings: the upstream
# gradient is a per-token weight dloss_n (1/N for the mean loss); masked padding columns have
# zero probability and so zero gradient; rank r's share of the logits gradient uses the merged
# (all-rank) per-token max M and sum S = sum_v exp(y_v - M), which is what the forward's
# exchange leaves on every rank.
# ------------------------------------------------------------------------------------------
def xent_full_grad(X, E, targets, Vreal, mask_padding=False, dloss=None):
    """Unsplit gradients of sum_n dloss_n * loss_n: dlogits = dloss * (softmax(y) - onehot),
    dX = dlogits E, dE = dlogits^T X (y = X E^T)."""
    N = X.shape[0]
    if dloss is None:
        dloss = np.full(N, 1.0 / N)
    y = _masked_logits(X, E, 0, Vreal, mask_padding)
    m = y.max(axis=1, keepdims=True)
    p = np.exp(y - m)
    p = p / p.sum(axis=1, keepdims=True)
    onehot = np.zeros_like(p)
    onehot[np.arange(N), targets] = 1.0
    dl = dloss[:, None] * (p - onehot)
    return {"dlogits": dl, "dX": dl @ E, "dE": dl.T @ X}


def xent_shard_grad(X, E_r, targets, t, r, Vreal, mask_padding, M, S, dloss):
    """Rank r's share given the merged per-token max M and sum S (over every rank's columns):
    dlogits_r = dloss * (exp(y_r - M) / S - onehot on the rank's columns), dX_r = dlogits_r E_r
    (a partial; the sum over ranks is dX) and dE_r = dlogits_r^T X (rank r's rows of dE)."""
    N, Vt = X.shape[0], E_r.shape[0]
    col0 = r * Vt
    y = _masked_logits(X, E_r, col0, Vreal, mask_padding)
    p = np.exp(y - M[:, None]) / S[:, None]
    local = targets.astype(np.int64) - col0
    owned = (local >= 0) & (local < Vt)
    onehot = np.zeros_like(p)
    n = np.arange(N)
    onehot[n[owned], local[owned]] = 1.0
    dl = dloss[:, None] * (p - onehot)
    return {"dlogits": dl, "dX": dl @ E_r, "dE": dl.T @ X}


def xent_merged_stats(X, E, targets, Vreal, mask_padding=False):
    """The merged per-token max M and sum S = sum_v exp(y_v - M) over the whole vocabulary
    (what the forward exchange yields on every rank)."""
    y = _masked_logits(X, E, 0, Vreal, mask_padding)
    M = y.max(axis=1)
    return M, np.exp(y - M[:, None]).sum(axis=1)
