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
GELU_CLAMP = 100.0                      # input clamp before the cube


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
    xc = np.clip(x, -GELU_CLAMP, GELU_CLAMP)
    inner = SQRT_2_OVER_PI * (xc + GELU_COEFF * xc ** 3)
    return 0.5 * x * (1.0 + np.tanh(inner))


def gelu_derivative(x_in):
    x = np.clip(np.asarray(x_in, dtype=np.float64), -GELU_CLAMP, GELU_CLAMP)
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
    x = np.clip(np.asarray(pre_gelu, dtype=np.float64), -GELU_CLAMP, GELU_CLAMP)
    with np.errstate(invalid="ignore", over="ignore"):
        return _gelu_backward(g, x, pre_gelu)


def _gelu_backward(g, x, pre_gelu):
    inner = SQRT_2_OVER_PI * (x + GELU_COEFF * x ** 3)
    t = np.tanh(inner)
    sech2 = 1.0 - t * t
    d_inner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_COEFF * x * x)
    im = _inner_mag(x)
    # 0.5 (1 + t): t's rounding, and the argument's (sech^2 times a few ulps
    # of |inner|); 0.5 x sech^2 d_inner: sech^2 = 1 - t^2 is computed with an
    # absolute error of a few ulps of 1 while tanh is short of +-1 in fp32,
    # and exactly (0) once it is +-1, which happens where the true sech^2
    # falls far below 2^-24: the floor is weighted by _unsaturated(sech^2).
    mag = np.abs(g) * (0.5 * (1.0 + np.abs(t)) * (1.0 + sech2 * im)
                       + 0.5 * np.abs(x) * d_inner * (sech2 * (1.0 + im) + SECH2_FLOOR * _unsaturated(sech2)))
    return nan_guard(g * gelu_derivative(pre_gelu)), nan_guard(mag)


def _unsaturated(sech2):
    """1 where fp32 tanh may still be an ulp short of +-1, falling to 0 with
    sech^2 beyond.  A correctly rounded tanh reaches +-1 once sech^2 is
    below about 2^-24; a faithfully rounded one (1 ulp) can stay an ulp
    short a little further (numpy's float32 tanh does so at |inner| = 10,
    sech^2 = 8e-9), so the floor is kept whole down to sech^2 = 2^-36
    (|inner| about 13) and decays with sech^2 below that.  At |x| >= 9
    (|inner| >= 33) it is below 1e-17."""
    return np.minimum(1.0, sech2 * 2.0 ** 36)


def _inner_mag(x):
    """|x| + 0.044715 |x|^3, scaled as the tanh argument: the size that the
    argument's own rounding is relative to."""
    return SQRT_2_OVER_PI * (np.abs(x) + GELU_COEFF * np.abs(x) ** 3)


def gelu_inplace(x):
    """(gelu(x), scale).  The scale collapses with 1 + t where tanh
    saturates at -1 (the result is 0 there, exactly in fp32 too): 1 + t is
    short by t's rounding only while fp32 tanh is not yet -1."""
    x64 = np.asarray(x, dtype=np.float64)
    xc = np.clip(x64, -GELU_CLAMP, GELU_CLAMP)
    t = np.tanh(SQRT_2_OVER_PI * (xc + GELU_COEFF * xc ** 3))
    sech2 = 1.0 - t * t
    scale = 0.5 * np.abs(x64) * ((1.0 + t) + sech2 * _inner_mag(xc) + T_FLOOR * _unsaturated(sech2))
    return gelu(x64), scale


# |x - x_ref| <= rel * scale + abs.  The scales are the magnitudes of the
# terms before they cancel, not of the result: in fp32 the page's GeLU
# formulas lose relative accuracy where tanh(inner) is within a few ulps of
# +-1, because 1 + t and 1 - t^2 cancel; there the error is a few ulps of 1
# in those differences (the floors below, in units of rel: 1e-6 for
# 1 - t^2, 5e-7 for 1 + t, about eight and four ulps of 1), times the
# factor they are multiplied by.  Where fp32 tanh is exactly +-1 both
# differences are exact and the floors vanish, so saturated inputs are held
# to the result itself.  Likewise silu' near its zero.  With fp32 exp and
# tanh good to about 2 ulps, 1e-5 leaves a margin of about ten elsewhere.
TOL = (1e-5, 1e-30)
SECH2_FLOOR = 1e-6 / TOL[0]
T_FLOOR = 5e-7 / TOL[0]
