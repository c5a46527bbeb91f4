"""MLP block, unsplit and t-way split, forward and backward, float64.

Test infrastructure only (see the package header).

Passages followed:
* forward, unsplit: "Megatron-LM: Training ... Model Parallelism" (paper digest), §3.4,
  "Column-Parallel GEMM for the First MLP Layer" (Y = GeLU(XA)) and "Row-Parallel GEMM for
  the Second MLP Layer" (Z = Y'B);
* split: same section, Option 2 (A cut by columns, each GPU applies GeLU to its own column
  block) and the row cut of B (each GPU's Z_i is a full-size partial; Z is their sum);
* backward: "Tensor and pipeline parallelism, and choosing a layout", §3, Proposition
  (Megatron MLP split), proof steps 4 and 5 (dB_i = Y_i^T G, dY_i = G B_i^T,
  dU_i = dY_i * GeLU'(U_i), dA_i = X^T dU_i, dX = sum_i dU_i A_i^T).

Biases: the pages' equations have none. The column-parallel bias b1 is cut with A's columns
and added before GeLU; the row-parallel bias b2 is added once, after the sum of partials
(adding it per shard would add it t times).

Pins: the 2x2 worked examples of "Megatron-LM, annotated" §3.1 (tests/golden); split equals
unsplit (forward and every gradient) to ~1e-12 relative; the partial dX_0 differs from dX;
PyTorch float64 autograd of the unsplit block; central finite differences.
"""
import numpy as np

from .gelu import gelu, gelu_grad


def shard_cols(W, t, r):
    """Rank r's column block of W: columns [r*n/t, (r+1)*n/t)."""
    n = W.shape[-1]
    assert n % t == 0
    w = n // t
    return W[..., r * w:(r + 1) * w]


def shard_rows(W, t, r):
    """Rank r's row block of W: rows [r*n/t, (r+1)*n/t)."""
    n = W.shape[0]
    assert n % t == 0
    w = n // t
    return W[r * w:(r + 1) * w]


def mlp_fwd(X, A, b1, B, b2):
    """Unsplit block: U = XA + b1, Y = GeLU(U), Z = YB + b2."""
    U = X @ A + b1
    Y = gelu(U)
    Z = Y @ B + b2
    return {"U": U, "Y": Y, "Z": Z}


def mlp_bwd(X, A, B, U, Y, G):
    """Unsplit backward for G = dL/dZ."""
    dY = G @ B.T
    dU = dY * gelu_grad(U)
    return {
        "dX": dU @ A.T,
        "dA": X.T @ dU,
        "db1": dU.sum(axis=0),
        "dB": Y.T @ G,
        "db2": G.sum(axis=0),
    }


def mlp_shard_fwd(X, A_r, b1_r, B_r):
    """One rank: U_r = X A_r + b1_r, Y_r = GeLU(U_r), Z_r = Y_r B_r (partial, no b2)."""
    U = X @ A_r + b1_r
    Y = gelu(U)
    return {"U": U, "Y": Y, "Z": Y @ B_r}


def mlp_shard_bwd(X, A_r, B_r, U_r, Y_r, G):
    """One rank's backward: local weight gradients and the partial dX_r (f sums them)."""
    dU = (G @ B_r.T) * gelu_grad(U_r)
    return {
        "dU": dU,
        "dX": dU @ A_r.T,
        "dA": X.T @ dU,
        "db1": dU.sum(axis=0),
        "dB": Y_r.T @ G,
    }


def mlp_split_fwd(X, A, b1, B, b2, t):
    """All t ranks, then the g sum: Z = sum_r Z_r + b2. Returns Z and the per-rank dicts."""
    ranks = [mlp_shard_fwd(X, shard_cols(A, t, r), shard_cols(b1, t, r), shard_rows(B, t, r))
             for r in range(t)]
    Z = sum(p["Z"] for p in ranks) + b2
    return {"Z": Z, "ranks": ranks}


def mlp_split_bwd(X, A, B, ranks_fwd, G, t):
    """All t ranks' backward, then the f sum of dX_r; weight gradients concatenated back."""
    ranks = [mlp_shard_bwd(X, shard_cols(A, t, r), shard_rows(B, t, r),
                           ranks_fwd[r]["U"], ranks_fwd[r]["Y"], G) for r in range(t)]
    return {
        "dX": sum(p["dX"] for p in ranks),
        "dA": np.concatenate([p["dA"] for p in ranks], axis=1),
        "db1": np.concatenate([p["db1"] for p in ranks]),
        "dB": np.concatenate([p["dB"] for p in ranks], axis=0),
        "db2": G.sum(axis=0),
        "ranks": ranks,
    }
