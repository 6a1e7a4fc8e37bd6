"""Activations that replace softmax in GDPA, and their derivatives, in fp64.

Test infrastructure (see the package docstring).

The GDPA README ("Features": custom activations) names GELU, GELUApprox,
FastGELU, FastGELU (BF16), ReLU, ReLU^2, LeakyReLU, SiLU, FastSiLU, HardSwish
and identity but gives no formulas.  The standard published definitions are
used:
  * GELU(x) = x * Phi(x), Phi the standard normal CDF (Hendrycks & Gimpel,
    "Gaussian Error Linear Units", 2016, eq. for GELU);
  * the tanh approximation of GELU from the same paper,
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)));
  * SiLU(x) = x * sigmoid(x);
  * HardSwish(x) = x * relu6(x + 3) / 6 (Howard et al., "Searching for
    MobileNetV3", 2019, eq. 2);
  * ReLU^2(x) = max(x, 0)^2; LeakyReLU(x) = x if x >= 0 else alpha x.
Reading: "GELUApprox", "FastGELU" and "FastGELU (BF16)" all denote the tanh
approximation (the jagged self-attention workload calls FastGELU "tanh GELU");
"FastSiLU" denotes SiLU.  The fast variants differ only in how a GPU evaluates
them, so the oracle evaluates the exact formula for every one of them.
Derivatives at kinks follow the PyTorch conventions (ReLU'(0) = 0,
LeakyReLU'(0) = alpha, HardSwish' = x/3 + 1/2 on [-3, 3]).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf, expit

ACT_NAMES = (
    "identity", "gelu", "gelu_tanh", "fast_gelu", "fast_gelu_bf16",
    "relu", "relu2", "leaky_relu", "silu", "fast_silu", "hardswish",
)

_SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)
_GELU_CUBIC = 0.044715
_TANH_GELU = ("gelu_tanh", "fast_gelu", "fast_gelu_bf16")


def _std_normal_pdf(x):
    return np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def act(name: str, x, alpha: float = 0.01):
    """act(x) elementwise in fp64."""
    x = np.asarray(x, dtype=np.float64)
    if name == "identity":
        return x.copy()
    if name == "gelu":
        return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))
    if name in _TANH_GELU:
        u = _SQRT_2_OVER_PI * (x + _GELU_CUBIC * x ** 3)
        return 0.5 * x * (1.0 + np.tanh(u))
    if name == "relu":
        return np.maximum(x, 0.0)
    if name == "relu2":
        r = np.maximum(x, 0.0)
        return r * r
    if name == "leaky_relu":
        return np.where(x >= 0.0, x, alpha * x)
    if name in ("silu", "fast_silu"):
        return x * expit(x)
    if name == "hardswish":
        return x * np.clip(x + 3.0, 0.0, 6.0) / 6.0
    raise ValueError(f"unknown activation {name!r}")


def act_grad(name: str, x, alpha: float = 0.01):
    """d act / dx elementwise in fp64."""
    x = np.asarray(x, dtype=np.float64)
    if name == "identity":
        return np.ones_like(x)
    if name == "gelu":
        return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * _std_normal_pdf(x)
    if name in _TANH_GELU:
        u = _SQRT_2_OVER_PI * (x + _GELU_CUBIC * x ** 3)
        t = np.tanh(u)
        du = _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_CUBIC * x * x)
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du
    if name == "relu":
        return (x > 0.0).astype(np.float64)
    if name == "relu2":
        return 2.0 * np.maximum(x, 0.0)
    if name == "leaky_relu":
        return np.where(x > 0.0, 1.0, alpha)
    if name in ("silu", "fast_silu"):
        s = expit(x)
        return s * (1.0 + x * (1.0 - s))
    if name == "hardswish":
        return np.where(x < -3.0, 0.0, np.where(x > 3.0, 1.0, x / 3.0 + 0.5))
    raise ValueError(f"unknown activation {name!r}")
