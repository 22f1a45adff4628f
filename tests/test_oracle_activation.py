"""Pins for the FFN activation oracle (oracle/activation.py), against values
fixed by something other than the oracle: the derivatives as central
differences of the forward functions (scipy's expit for silu; the tanh
approximation for gelu), closed forms at 0 and in the saturated tails,
scipy's expit for the sigmoid, the exact GeLU (x Phi(x)) to the known
accuracy of its tanh approximation, and nan_guard on NaN and infinities.
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


PINS = [check_sigmoid_silu, check_silu_derivative, check_gelu_and_derivative, check_chain_rules, check_nan_guard]


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
    "gelu_coeff": {"sech2 = 1.0 - t * t\n    d_inner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_COEFF * x * x)":
                   "sech2 = 1.0 - t * t\n    d_inner = SQRT_2_OVER_PI * (1.0 + GELU_COEFF * x * x)"},
    "grad_up_uses_gate": {"du = nan_guard(g * silu(x))": "du = nan_guard(g * x)"},
    "no_nan_guard": {"return np.where(np.isfinite(x), x, 0.0)": "return x"},
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
