"""Pins for the fused-loss oracle (oracle/loss.py), against values fixed by
something other than the oracle: closed forms (uniform logits, two classes),
scipy's logsumexp and softmax, the gradient as the numerical derivative of
the loss (central differences in float64, with label smoothing and z-loss),
the sum of a gradient row (2 beta lse inv_norm, since p and the target each
sum to one), ignored rows, and math.fsum for sum_losses.  The last test runs
the pins against planted mistakes."""
import math
import types

import numpy as np
import pytest

from oracle import loss as L


def check_uniform(orc):
    V = 1000
    for a in (0.0, 0.1):
        logits = np.full((2, V), 3.25, dtype=np.float32)
        loss, dl, _ = orc.cross_entropy(logits, np.array([7, 999]), alpha=a, inv_norm=0.5)
        assert np.allclose(loss, math.log(V), rtol=1e-14, atol=0)
        want = np.full(V, 1.0 / V) - a / V
        want[7] -= 1.0 - a
        assert np.allclose(dl[0], want * 0.5, rtol=0, atol=1e-15)


def check_two_class(orc):
    a, b = 1.5, -0.75
    loss, dl, _ = orc.cross_entropy(np.array([[a, b]], np.float32), np.array([0]))
    assert abs(loss[0] - math.log1p(math.exp(b - a))) < 1e-14
    sig = 1.0 / (1.0 + math.exp(-(a - b)))
    assert abs(dl[0, 0] - (sig - 1.0)) < 1e-14 and abs(dl[0, 1] - (1.0 - sig)) < 1e-14


def check_scipy(orc, seed=30):
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(seed)
    S, V = 6, 777
    logits = (rng.standard_normal((S, V)) * 4).astype(np.float32)
    tg = rng.integers(0, V, S)
    loss, dl, _ = orc.cross_entropy(logits, tg, inv_norm=1.0 / S)
    l64 = logits.astype(np.float64)
    want = logsumexp(l64, axis=1) - l64[np.arange(S), tg]
    assert np.allclose(loss, want, rtol=1e-13, atol=1e-13)
    g = softmax(l64, axis=1)
    g[np.arange(S), tg] -= 1.0
    assert np.allclose(dl, g / S, rtol=1e-12, atol=1e-16)


def check_gradient_is_derivative(orc, seed=31):
    rng = np.random.default_rng(seed)
    V = 40
    for (a, b) in [(0.0, 0.0), (0.1, 0.0), (0.0, 0.05), (0.2, 0.3)]:
        l = (rng.standard_normal(V) * 2).astype(np.float32)
        tgt = int(rng.integers(0, V))
        _, dl, _ = orc.cross_entropy(l[None], np.array([tgt]), alpha=a, beta=b, inv_norm=1.0)

        def f(x):   # the loss as a function of float64 logits, through the oracle
            ls, _, _ = orc.cross_entropy(x[None], np.array([tgt]), alpha=a, beta=b)
            return ls[0]
        x0 = l.astype(np.float64)
        h = 1e-5
        for v in range(V):
            xp, xm = x0.copy(), x0.copy()
            xp[v] += h
            xm[v] -= h
            num = (f(xp) - f(xm)) / (2 * h)
            assert abs(num - dl[0, v]) <= 1e-7, (a, b, v, num, dl[0, v])


def check_row_sums_and_ignore(orc, seed=32):
    rng = np.random.default_rng(seed)
    S, V = 5, 300
    logits = (rng.standard_normal((S, V)) * 3).astype(np.float32)
    tg = np.array([0, V - 1, V, 2 ** 32 - 1, 17], dtype=np.uint32)   # rows 2 and 3 ignored
    for (a, b, inv) in [(0.0, 0.0, 0.25), (0.1, 1e-4, 1.0 / 3)]:
        loss, dl, _ = orc.cross_entropy(logits, tg, alpha=a, beta=b, inv_norm=inv)
        assert loss[2] == 0.0 and loss[3] == 0.0 and not dl[2].any() and not dl[3].any()
        for r in (0, 1, 4):
            l = logits[r].astype(np.float64)
            lse = l.max() + math.log(np.exp(l - l.max()).sum())
            assert abs(dl[r].sum() - 2 * b * lse * inv) <= 1e-12
            assert loss[r] > 0.0


def check_sum_losses(orc, seed=33):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(4099) * 1e3).astype(np.float32)
    assert orc.sum_losses(x) == math.fsum(float(v) for v in x)
    assert orc.sum_losses(np.zeros(0, np.float32)) == 0.0


PINS = [check_uniform, check_two_class, check_scipy, check_gradient_is_derivative, check_row_sums_and_ignore,
        check_sum_losses]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_loss_pins(pin):
    pin(L)


def _mutant(**patch):
    """A copy of the oracle module's functions with one formula changed."""
    import inspect
    src = inspect.getsource(L)
    for old, new in patch.items():
        assert src.count(old) == 1, old
        src = src.replace(old, new)
    ns = {}
    exec(compile(src, "loss_mutant", "exec"), ns)
    return types.SimpleNamespace(**ns)


MUTANTS = {
    "alpha_sign": {"- alpha * mean_l": "+ alpha * mean_l"},
    "zloss_grad_factor": {"2.0 * beta * lse * p": "beta * lse * p"},
    "no_max_shift_in_p": {"p = e / denom": "p = np.exp(l) / denom"},
    "smoothing_mass": {"target = np.full(V, alpha / V)": "target = np.full(V, alpha)"},
    "ignore_keeps_row": {"        if tgt >= V:\n            continue": "        if tgt >= V + 1:\n            continue"},
    "sum_drops_last": {"for x in np.asarray(losses, dtype=np.float64))": "for x in np.asarray(losses, dtype=np.float64)[:-1])"},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_loss_mistakes_are_caught(name):
    m = _mutant(**MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"
