"""Replicated LayerNorm, forward and backward, float64.

Test infrastructure only (see the package header).

Passage: "Megatron-LM: Training ... Model Parallelism" (paper digest), §3.4, "Duplicate
Computation vs. Communication: Dropout, Layer Normalization, and Residual Connections":
every GPU keeps its own copy of the norm's gain and shift and normalises its own copy of
the activations; "Megatron-LM, annotated", §3.5 (the norm has 2H parameters).
The pages give no constants. Readings: statistics over the hidden dimension, biased
variance (divide by h), eps = 1e-5, y = (x - mean) / sqrt(var + eps) * gain + shift.
Backward is the textbook chain rule.

Pins: PyTorch CPU float64 layer_norm and its autograd; with gain 1 and shift 0 each row has
mean 0 and variance var/(var+eps); central finite differences.
"""
import numpy as np

EPS = 1e-5


def layernorm_fwd(x, gamma, beta, eps=EPS):
    mean = x.mean(axis=1)
    var = ((x - mean[:, None]) ** 2).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean[:, None]) * rstd[:, None]
    return {"y": xhat * gamma + beta, "mean": mean, "rstd": rstd}


def layernorm_bwd(x, gamma, mean, rstd, dy):
    h = x.shape[1]
    xhat = (x - mean[:, None]) * rstd[:, None]
    g = dy * gamma
    dx = rstd[:, None] * (g - g.mean(axis=1, keepdims=True)
                          - xhat * (g * xhat).sum(axis=1, keepdims=True) / h)
    return {"dx": dx, "dgamma": (dy * xhat).sum(axis=0), "dbeta": dy.sum(axis=0)}
