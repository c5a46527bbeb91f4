"""Self-attention block, unsplit and head-sharded, forward and backward, float64.

Test infrastructure only (see the package header).

Passages followed:
* "Megatron-LM: Training ... Model Parallelism" (paper digest), §3.4, "Attention Head
  Parallelism in the Self-Attention Block": the Q, K, V projections are cut by columns
  along whole heads; each GPU runs softmax(query_i key_i^T / sqrt(d_k)) value_i for its own
  heads; the output projection O is cut by rows and the partials are summed (g);
* "Megatron-LM, annotated", §2.2 (GPT-2 is a decoder that writes left to right, hence the
  causal mask) and §3.2 The attention block (8.3B model: 32 heads, 4 per GPU, width 96);
* backward: not on the pages. It is the textbook chain rule through S = QK^T*c,
  P = softmax(S), O = PV: dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)),
  dQ = c dS K, dK = c dS^T Q.

Layouts (readings where the pages are silent): tokens are rows, token = batch*s + position.
The full projection Wqkv is [h, 3h] = [Wq | Wk | Wv], head j owning columns j*d..(j+1)*d of
each third. Rank r owns the contiguous heads r*a/t .. (r+1)*a/t - 1, so its packed weight is
[Wq[:, H_r] | Wk[:, H_r] | Wv[:, H_r]] of shape [h, 3h/t], and its output-projection rows are
Wo[H_r, :]. The scale is 1/sqrt(d) with d the head width. Query i sees keys j <= i of its own
sequence. lse is the natural log of the row's sum of exp of the scaled, masked scores.

Pins: PyTorch CPU float64 scaled_dot_product_attention (causal and not) for the core;
s = 1 gives O = V; Q = 0 gives the running mean of V (closed form); future tokens do not
change past outputs (causality); sum of head-sharded partials equals the unsplit block;
t = 1 equals the unsplit block; float64 autograd and central finite differences for the
backward.
"""
import math

import numpy as np


def head_columns(h, heads, t, r):
    """Column range [lo, hi) of rank r's heads inside one of the Q/K/V thirds."""
    assert heads % t == 0 and h % heads == 0
    ht = h // t
    return r * ht, (r + 1) * ht


def qkv_shard(Wqkv, heads, t, r):
    """Rank r's packed [Wq_r | Wk_r | Wv_r] from the full [h, 3h] projection (or its bias)."""
    h = Wqkv.shape[-1] // 3
    lo, hi = head_columns(h, heads, t, r)
    parts = [Wqkv[..., i * h + lo:i * h + hi] for i in range(3)]
    return np.concatenate(parts, axis=-1)


def wo_shard(Wo, heads, t, r):
    """Rank r's rows of the output projection."""
    h = Wo.shape[0]
    lo, hi = head_columns(h, heads, t, r)
    return Wo[lo:hi]


def attn_core_fwd(Q, K, V, causal, keep=None, scale=1.0):
    """One (sequence, head): S = QK^T/sqrt(d), masked, P = softmax(S), O = PV, lse per row.

    With a dropout keep mask (the paper digest's "dropout within attention", §3.4, applied to the
    attention weights): O = (P * keep * scale) V; P and lse stay those of the undropped softmax."""
    s, d = Q.shape
    S = (Q @ K.T) / math.sqrt(d)
    if causal:
        S = np.where(np.tril(np.ones((s, s), dtype=bool)), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    denom = E.sum(axis=1, keepdims=True)
    P = E / denom
    Pd = P if keep is None else np.where(keep, P * scale, 0.0)
    return {"O": Pd @ V, "P": P, "lse": (m + np.log(denom))[:, 0]}


def attn_core_bwd(Q, K, V, P, dO, keep=None, scale=1.0):
    """Textbook backward of one (sequence, head) given the forward's P (and its dropout mask:
    with Pd = P * keep * scale, dV = Pd^T dO and dP = (dO V^T) * keep * scale)."""
    d = Q.shape[1]
    c = 1.0 / math.sqrt(d)
    Pd = P if keep is None else np.where(keep, P * scale, 0.0)
    dV = Pd.T @ dO
    dP = dO @ V.T
    if keep is not None:
        dP = np.where(keep, dP * scale, 0.0)
    dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
    return {"dQ": c * (dS @ K), "dK": c * (dS.T @ Q), "dV": dV}


def _split_qkv(QKV, nh, d):
    w = nh * d
    return QKV[:, :w], QKV[:, w:2 * w], QKV[:, 2 * w:3 * w]


def _keep_masks(drop, b, s, nh):
    """Dropout keep masks of a rank's heads: drop = {p, seed, stream, heads (all ranks), head0}."""
    if drop is None or drop["p"] == 0.0:
        return None
    from .rng import attn_keep
    return {(bi, j): attn_keep(bi, drop["head0"] + j, s, drop["heads"], drop["p"], drop["seed"], drop["stream"])
            for bi in range(b) for j in range(nh)}


def _heads_fwd(QKV, b, s, nh, d, causal, keep=None, scale=1.0):
    Q, K, V = _split_qkv(QKV, nh, d)
    T = b * s
    O = np.zeros((T, nh * d))
    lse = np.zeros((b, nh, s))
    P = {}
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            cols = slice(j * d, (j + 1) * d)
            out = attn_core_fwd(Q[rows, cols], K[rows, cols], V[rows, cols], causal,
                                None if keep is None else keep[bi, j], scale)
            O[rows, cols] = out["O"]
            lse[bi, j] = out["lse"]
            P[bi, j] = out["P"]
    return O, lse, P


def _heads_bwd(QKV, P, dO, b, s, nh, d, keep=None, scale=1.0):
    Q, K, V = _split_qkv(QKV, nh, d)
    dQKV = np.zeros_like(QKV)
    w = nh * d
    for bi in range(b):
        rows = slice(bi * s, (bi + 1) * s)
        for j in range(nh):
            cols = slice(j * d, (j + 1) * d)
            g = attn_core_bwd(Q[rows, cols], K[rows, cols], V[rows, cols], P[bi, j], dO[rows, cols],
                              None if keep is None else keep[bi, j], scale)
            dQKV[rows, j * d:(j + 1) * d] = g["dQ"]
            dQKV[rows, w + j * d:w + (j + 1) * d] = g["dK"]
            dQKV[rows, 2 * w + j * d:2 * w + (j + 1) * d] = g["dV"]
    return dQKV


def attn_shard_fwd(Xn, Wqkv_r, bqkv_r, Wo_r, b, s, heads_t, causal=True, drop=None):
    """One rank: QKV_r = Xn Wqkv_r + bqkv_r; attention for its heads; Z_r = O_r Wo_r (no bo).
    drop: attention dropout {p, seed, stream, heads, head0} (oracle.rng's mapping), or None."""
    d = Wo_r.shape[0] // heads_t
    QKV = Xn @ Wqkv_r + bqkv_r
    keep = _keep_masks(drop, b, s, heads_t)
    scale = 1.0
    if keep is not None:
        from .rng import drop_scale
        scale = drop_scale(drop["p"])
    O, lse, P = _heads_fwd(QKV, b, s, heads_t, d, causal, keep, scale)
    return {"QKV": QKV, "O": O, "lse": lse, "P": P, "Z": O @ Wo_r, "keep": keep, "scale": scale}


def attn_shard_bwd(Xn, Wqkv_r, Wo_r, fwd_r, G, b, s, heads_t):
    """One rank's backward for G = dL/dZ: dWo_r, the attention chain, dWqkv_r, dbqkv_r and
    the partial dXn_r (f sums the ranks' partials)."""
    d = Wo_r.shape[0] // heads_t
    dO = G @ Wo_r.T
    dQKV = _heads_bwd(fwd_r["QKV"], fwd_r["P"], dO, b, s, heads_t, d, fwd_r.get("keep"), fwd_r.get("scale", 1.0))
    return {
        "dO": dO,
        "dQKV": dQKV,
        "dWo": fwd_r["O"].T @ G,
        "dWqkv": Xn.T @ dQKV,
        "dbqkv": dQKV.sum(axis=0),
        "dXn": dQKV @ Wqkv_r.T,
    }


def attn_fwd(Xn, Wqkv, bqkv, Wo, bo, b, s, heads, causal=True):
    """Unsplit block: every head of the full projection, Z = O Wo + bo."""
    h = Wo.shape[0]
    d = h // heads
    QKV = Xn @ Wqkv + bqkv
    O, lse, P = _heads_fwd(QKV, b, s, heads, d, causal)
    return {"QKV": QKV, "O": O, "lse": lse, "P": P, "Z": O @ Wo + bo}


def attn_bwd(Xn, Wqkv, Wo, fwd, G, b, s, heads):
    """Unsplit backward."""
    h = Wo.shape[0]
    d = h // heads
    dO = G @ Wo.T
    dQKV = _heads_bwd(fwd["QKV"], fwd["P"], dO, b, s, heads, d)
    return {
        "dXn": dQKV @ Wqkv.T,
        "dWqkv": Xn.T @ dQKV,
        "dbqkv": dQKV.sum(axis=0),
        "dWo": fwd["O"].T @ G,
        "dbo": G.sum(axis=0),
    }


def attn_split_fwd(Xn, Wqkv, bqkv, Wo, bo, b, s, heads, t, causal=True, drop=None):
    """All t ranks, then the g sum: Z = sum_r Z_r + bo. drop: {p, seed, streams[t]} (rank r's
    attention dropout uses streams[r]) or None."""
    def rank_drop(r):
        if drop is None:
            return None
        return {"p": drop["p"], "seed": drop["seed"], "stream": drop["streams"][r], "heads": heads,
                "head0": r * (heads // t)}
    ranks = [attn_shard_fwd(Xn, qkv_shard(Wqkv, heads, t, r), qkv_shard(bqkv, heads, t, r),
                            wo_shard(Wo, heads, t, r), b, s, heads // t, causal, rank_drop(r))
             for r in range(t)]
    return {"Z": sum(p["Z"] for p in ranks) + bo, "ranks": ranks}


def attn_split_bwd(Xn, Wqkv, Wo, ranks_fwd, G, b, s, heads, t):
    """All t ranks' backward, the f sum of dXn_r, and the weight gradients put back in the
    full layout."""
    ranks = [attn_shard_bwd(Xn, qkv_shard(Wqkv, heads, t, r), wo_shard(Wo, heads, t, r),
                            ranks_fwd[r], G, b, s, heads // t) for r in range(t)]
    h = Wo.shape[0]
    dWqkv = np.zeros_like(Wqkv)
    dbqkv = np.zeros(3 * h)
    dWo = np.zeros_like(Wo)
    for r, g in enumerate(ranks):
        lo, hi = head_columns(h, heads, t, r)
        w = hi - lo
        for i in range(3):
            dWqkv[:, i * h + lo:i * h + hi] = g["dWqkv"][:, i * w:(i + 1) * w]
            dbqkv[i * h + lo:i * h + hi] = g["dbqkv"][i * w:(i + 1) * w]
        dWo[lo:hi] = g["dWo"]
    return {"dXn": sum(g["dXn"] for g in ranks), "dWqkv": dWqkv, "dbqkv": dbqkv, "dWo": dWo,
            "dbo": G.sum(axis=0), "ranks": ranks}
