"""GeLU and its derivative, float64. Test infrastructure only (see the package header).

Definition: "Megatron-LM, annotated", §2.2 Transformer language models and multi-head
attention: GELU(x) is x times the standard normal CDF at x, written with the error function.
The lesson page "Tensor and pipeline parallelism, and choosing a layout" (§5, "In code")
uses the tanh approximation instead; the erf form is the one the printed values fix
(GELU(2) rounds to 1.954 only for erf; tanh gives 1.9546).

Pins: printed values GELU(1), GELU(-1), GELU(2) and the implied GELU(-2) (tests/golden);
PyTorch CPU float64 ``gelu`` (exact form); central finite differences for ``gelu_grad``;
the limits GELU(x) -> x, GELU'(x) -> 1 for large x and -> 0 for very negative x.
"""
import math

import numpy as np
from scipy.special import erf

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def gelu(x):
    """x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2, elementwise, float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / _SQRT2))


def gelu_grad(x):
    """d/dx [x * Phi(x)] = Phi(x) + x * phi(x), phi the standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    cdf = 0.5 * (1.0 + erf(x / _SQRT2))
    pdf = _INV_SQRT_2PI * np.exp(-0.5 * x * x)
    return cdf + x * pdf


def gelu_scalar(x: float) -> float:
    """Pure-Python scalar GeLU for the pages' worked examples."""
    return x * 0.5 * (1.0 + math.erf(x / _SQRT2))
