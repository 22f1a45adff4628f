"""Pins for the FFN activation oracle (oracle/activation.py), against values
fixed by something other than the oracle: the derivatives as central
differences of the forward functions (scipy's expit for silu; the tanh
approximation for gelu), closed forms at 0 and in the saturated tails,
scipy's expit for the sigmoid, the exact GeLU (x Phi(x)) to the known
accuracy of its tanh approximation, the GeLU constants as the page prints
them (tests/golden/gelu_constants.txt), the saturated tails exactly, the
tolerance against the page's formulas evaluated in fp32, and nan_guard on
NaN and infinities.
The last test runs the pins against planted mistakes."""
import math
import types

import numpy as np
import pytest

from oracle import activation as A


def check_sigmoid_silu(orc):
    from scipy.special import expit
    x = np.concatenate([np.linspace(-30, 30, 601), [-800.0, 800.0, 0.0]])
    assert np.allclose(orc.sigmoid(x), expit(x), rtol=1e-15, atol=0)
    assert np.allclose(orc.silu(x), x * expit(x), rtol=1e-15, atol=0)


def check_silu_derivative(orc):
    from scipy.special import expit
    x = np.linspace(-12, 12, 241)
    h = 1e-6
    num = ((x + h) * expit(x + h) - (x - h) * expit(x - h)) / (2 * h)
    assert np.allclose(orc.silu_derivative(x), num, rtol=0, atol=1e-8)
    assert orc.silu_derivative(0.0) == 0.5
    assert abs(orc.silu_derivative(-1.2784645427610738)) < 1e-12   # the derivative's zero


def check_gelu_and_derivative(orc):
    x = np.linspace(-8, 8, 321)
    c = math.sqrt(2 / math.pi)
    ref = 0.5 * x * (1 + np.tanh(c * (x + 0.044715 * x ** 3)))
    assert np.allclose(orc.gelu(x), ref, rtol=1e-15, atol=1e-300)
    # the tanh form approximates the exact x Phi(x) to about 1e-3
    from scipy.special import ndtr
    assert np.max(np.abs(orc.gelu(x) - x * ndtr(x))) < 1e-3
    h = 1e-6
    num = (orc.gelu(x + h) - orc.gelu(x - h)) / (2 * h)
    assert np.allclose(orc.gelu_derivative(x), num, rtol=0, atol=1e-8)
    assert orc.gelu_derivative(0.0) == 0.5
    assert orc.gelu_derivative(150.0) == 1.0 and orc.gelu_derivative(-150.0) == 0.0
    assert orc.gelu(-150.0) == 0.0 and orc.gelu(150.0) == 150.0


def check_chain_rules(orc, seed=40):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(500)
    x = rng.standard_normal(500) * 4
    u = rng.standard_normal(500)
    dg, du, _, _ = orc.ffn_swiglu_backward(g, x, u)
    h = 1e-6
    hid = lambda xx, uu: orc.silu(xx) * uu   # forward: hidden = silu(gate) * up
    assert np.allclose(dg, g * (hid(x + h, u) - hid(x - h, u)) / (2 * h), rtol=0, atol=1e-7)
    assert np.allclose(du, g * (hid(x, u + h) - hid(x, u - h)) / (2 * h), rtol=0, atol=1e-7)
    dp, _ = orc.ffn_gelu_backward(g, x)
    assert np.allclose(dp, g * (orc.gelu(x + h) - orc.gelu(x - h)) / (2 * h), rtol=0, atol=1e-7)


def check_nan_guard(orc):
    g = np.array([1.0, np.nan, 2.0, 1.0, np.inf])
    x = np.array([0.5, 0.5, np.nan, np.inf, 0.5])
    u = np.array([1.0, 1.0, 1.0, 1.0, 1.0])
    dg, du, _, _ = orc.ffn_swiglu_backward(g, x, u)
    assert np.all(np.isfinite(dg)) and np.all(np.isfinite(du))
    assert dg[1] == 0.0 and du[1] == 0.0 and dg[2] == 0.0 and dg[4] == 0.0
    dp, _ = orc.ffn_gelu_backward(g, x)
    assert np.all(np.isfinite(dp)) and dp[1] == 0.0 and dp[4] == 0.0
    assert dp[3] == 1.0 * orc.gelu_derivative(100.0)    # an infinite input is clamped first


def _golden_constants():
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gelu_constants.txt")
    out = {}
    with open(path) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value = line.split()
                out[name] = value
    return out


def check_gelu_constants_as_printed(orc):
    """The GeLU constants are the values the page prints (golden fixture):
    the oracle's cubic coefficient, inner scale and clamp, and gelu' at a
    point against the same formula taken with the printed constants."""
    k = _golden_constants()
    assert orc.GELU_COEFF == float(k["cubic_coefficient"])
    assert k["inner_scale"] == "sqrt(2/pi)" and orc.SQRT_2_OVER_PI == math.sqrt(2.0 / math.pi)
    clamp = float(k["clamp"])
    assert orc.GELU_CLAMP == clamp
    c = float(k["cubic_coefficient"])
    # the clamp: beyond it the derivative and the cube use +-100
    assert orc.gelu_derivative(1e6) == orc.gelu_derivative(clamp)
    assert orc.gelu_derivative(-1e6) == orc.gelu_derivative(-clamp)
    # a point where the coefficient matters to 1e-3 relative: x = 1.7,
    # inner = sqrt(2/pi) (1.7 + c 1.7^3); gelu' from the printed constants
    x = 1.7
    inner = math.sqrt(2 / math.pi) * (x + c * x ** 3)
    t = math.tanh(inner)
    expect = 0.5 * (1 + t) + 0.5 * x * (1 - t * t) * math.sqrt(2 / math.pi) * (1 + 3 * c * x * x)
    assert abs(float(orc.gelu_derivative(x)) - expect) <= 1e-15


def check_gelu_saturated_tails(orc):
    """Where tanh is +-1 in double precision (|x| >= 9: |inner| >= 33) the
    derivative is exactly 1 or 0 and gelu exactly x or 0, and the tolerance
    scales collapse to the result: a 0 for 1 swap fails by 1e5 bounds."""
    xs = np.array([9.0, 20.0, 50.0, 100.0, 200.0, 1e30])
    g = np.array([1.5, -2.0, 0.25, 3.0, -1.0, 7.0])
    for sign, want in ((1.0, 1.0), (-1.0, 0.0)):
        x = sign * xs
        assert np.all(orc.gelu_derivative(x) == want)
        d, m = orc.ffn_gelu_backward(g, x)
        assert np.all(d == g * want)
        assert np.all(m <= np.abs(g) * (1.0 + 1e-12))          # the bound is 1e-5 |g|, not |g| |x|^3
        wrong = g * (1.0 - want)
        assert np.all(np.abs(wrong - d) > orc.TOL[0] * m * 1e4)
        y, s = orc.gelu_inplace(x)
        assert np.all(y == (x if want else 0.0))
        assert np.all(s <= np.abs(y) + 1e-300)                  # relative to the result itself


def check_gelu_tolerance_covers_fp32(orc):
    """The page's formulas evaluated in fp32 (numpy float32, tanh faithfully
    rounded) stay within half the bound on a dense grid over the clamp range,
    while a 1% error in the cubic coefficient of the same fp32 evaluation
    fails on most of it: the bound is as loose as fp32 needs, no looser."""
    f = np.float32
    x = np.concatenate([np.linspace(-12, 12, 48001), np.linspace(-100, 100, 4001)]).astype(f)
    g = np.ones_like(x)

    def fp32(coeff):
        c, a = f(math.sqrt(2 / math.pi)), f(coeff)
        xc = np.clip(x, f(-100), f(100))
        x2 = xc * xc
        t = np.tanh(c * (xc + a * x2 * xc)).astype(f)
        d = f(0.5) * (f(1) + t) + f(0.5) * xc * (f(1) - t * t) * (c * (f(1) + f(3) * a * x2))
        return d, f(0.5) * x * (f(1) + t)

    ref_d, m = orc.ffn_gelu_backward(g, x)
    ref_y, s = orc.gelu_inplace(x)
    d, y = fp32(0.044715)
    assert np.max(np.abs(d - ref_d) / (orc.TOL[0] * m + orc.TOL[1])) <= 0.5
    assert np.max(np.abs(y - ref_y) / (orc.TOL[0] * s + orc.TOL[1])) <= 0.5
    d, y = fp32(0.044715 * 1.01)
    live = np.abs(x) <= 6          # beyond, tanh is +-1 whatever the coefficient
    assert np.mean((np.abs(d - ref_d) > orc.TOL[0] * m + orc.TOL[1])[live]) > 0.3


PINS = [check_sigmoid_silu, check_silu_derivative, check_gelu_and_derivative, check_chain_rules, check_nan_guard,
        check_gelu_constants_as_printed, check_gelu_saturated_tails, check_gelu_tolerance_covers_fp32]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_activation_pins(pin):
    pin(A)


def _mutant(**patch):
    import inspect
    src = inspect.getsource(A)
    for old, new in patch.items():
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    ns = {}
    exec(compile(src, "activation_mutant", "exec"), ns)
    return types.SimpleNamespace(**ns)


MUTANTS = {
    "silu_prime_sign": {"return s * (1.0 + x * (1.0 - s))": "return s * (1.0 - x * (1.0 - s))"},
    "sigmoid_branch": {"e / (1.0 + e))": "1.0 / (1.0 + e))"},
    "gelu_coeff": {"d_inner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_COEFF * x * x)\n    return 0.5":
                   "d_inner = SQRT_2_OVER_PI * (1.0 + GELU_COEFF * x * x)\n    return 0.5"},
    "grad_up_uses_gate": {"du = nan_guard(g * silu(x))": "du = nan_guard(g * x)"},
    "no_nan_guard": {"return np.where(np.isfinite(x), x, 0.0)": "return x"},
    "gelu_coeff_typo": {"GELU_COEFF = 0.044715": "GELU_COEFF = 0.0447"},
    "gelu_tolerance_without_collapse": {"SECH2_FLOOR * _unsaturated(sech2)": "SECH2_FLOOR + _inner_mag(x)"},
    "gelu_clamp_50": {"GELU_CLAMP = 100.0": "GELU_CLAMP = 50.0"},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_activation_mistakes_are_caught(name):
    m = _mutant(**MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"
