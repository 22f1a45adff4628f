"""Reference oracle for the FFN activation kernels (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by the test suite and bench.py's CPU
baseline, never by the product path.

Follows "ffn_gelu_backward ve ffn_swiglu_backward — FFN Activation Backward"
(https://llm.istanbul/learn/tr/09_backward_ffn): section "Ne Yapar?" (the
chain rule for both), "Türevler" (gelu by its tanh approximation and its
derivative with x clamped to [-100, 100]; silu' = s (1 + x (1 - s)) with the
sign-branched sigmoid), "Satır Satır" (both gradients pass through
nan_guard), and the shared preamble's nan_guard ("00_shared" page: a
non-finite value becomes 0).  gelu_inplace is read from its name and the
derivative section: x becomes gelu(x), optionally keeping a copy of x.
Every step is plain numpy in float64.
"""
from __future__ import annotations

import numpy as np

SQRT_2_OVER_PI = 0.7978845608028654     # sqrt(2 / pi)
GELU_COEFF = 0.044715


def nan_guard(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.isfinite(x), x, 0.0)


def sigmoid(x):
    """The sign-branched sigmoid: exp only ever sees a non-positive argument."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def silu_derivative(x):
    x = np.asarray(x, dtype=np.float64)
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def gelu(x):
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); the cube is taken of
    x clamped to [-100, 100], where tanh is already +-1."""
    x = np.asarray(x, dtype=np.float64)
    xc = np.clip(x, -100.0, 100.0)
    inner = SQRT_2_OVER_PI * (xc + GELU_COEFF * xc ** 3)
    return 0.5 * x * (1.0 + np.tanh(inner))


def gelu_derivative(x_in):
    x = np.clip(np.asarray(x_in, dtype=np.float64), -100.0, 100.0)
    inner = SQRT_2_OVER_PI * (x + GELU_COEFF * x ** 3)
    t = np.tanh(inner)
    sech2 = 1.0 - t * t
    d_inner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_COEFF * x * x)
    return 0.5 * (1.0 + t) + 0.5 * x * sech2 * d_inner


def ffn_swiglu_backward(grad_hidden, gate, up):
    """(grad_gate, grad_up, scale_gate, scale_up): grad_gate = g u silu'(gate),
    grad_up = g silu(gate), each through nan_guard; the scales are the
    magnitudes the fp32 rounding is relative to."""
    g = np.asarray(grad_hidden, dtype=np.float64)
    x = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        s = sigmoid(x)
        dg = nan_guard(g * u * silu_derivative(x))
        du = nan_guard(g * silu(x))
        mg = np.abs(g * u) * s * (1.0 + np.abs(x) * (1.0 - s))
        mu = np.abs(g * x) * s
    return dg, du, nan_guard(mg), nan_guard(mu)


def ffn_gelu_backward(grad_hidden, pre_gelu):
    """(grad_pre, scale): grad_pre = nan_guard(g gelu'(pre))."""
    g = np.asarray(grad_hidden, dtype=np.float64)
    x = np.clip(np.asarray(pre_gelu, dtype=np.float64), -100.0, 100.0)
    with np.errstate(invalid="ignore", over="ignore"):
        return _gelu_backward(g, x, pre_gelu)


def _gelu_backward(g, x, pre_gelu):
    inner = SQRT_2_OVER_PI * (x + GELU_COEFF * x ** 3)
    t = np.tanh(inner)
    d_inner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_COEFF * x * x)
    mag = np.abs(g) * (1.0 + np.abs(x) * d_inner) * (1.0 + (1.0 - t * t) * _inner_mag(x))
    return nan_guard(g * gelu_derivative(pre_gelu)), nan_guard(mag)


def _inner_mag(x):
    """|x| + 0.044715 |x|^3, scaled as the tanh argument: the size that the
    argument's own rounding is relative to."""
    return SQRT_2_OVER_PI * (np.abs(x) + GELU_COEFF * np.abs(x) ** 3)


def gelu_inplace(x):
    """(gelu(x), scale)."""
    x64 = np.asarray(x, dtype=np.float64)
    xc = np.clip(x64, -100.0, 100.0)
    t = np.tanh(SQRT_2_OVER_PI * (xc + GELU_COEFF * xc ** 3))
    return gelu(x64), np.abs(x64) * (1.0 + (1.0 - t * t) * _inner_mag(xc))


# |x - x_ref| <= rel * scale + abs.  The scales are the magnitudes of the
# terms before they cancel, not of the result: in fp32 the page's GeLU
# formulas lose all relative accuracy where tanh(inner) is within an ulp of
# +-1 (|x| > ~4), because 1 + t and 1 - t^2 cancel; the error there is a few
# ulps of 0.5 (1 + |t|) and of 0.5 |x| (1 + t^2) d_inner, and the argument's
# rounding adds sech^2 times a few ulps of |inner|.  Likewise silu' near its
# zero.  With fp32 exp and tanh good to about 2 ulps, 1e-5 leaves a margin of
# about ten over the worst case.
TOL = (1e-5, 1e-30)
