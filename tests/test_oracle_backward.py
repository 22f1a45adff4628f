"""Pins for the oracle's backward linear family (matmul_t, matmul_at, their
_acc forms and matmul_at_swiglu_a), against values fixed by something other
than the oracle itself: exact integer arithmetic in Python, the adjoint
identities that tie them to the (separately pinned) forward product,
identity operands, and an independently formed SwiGLU activation (scipy's
expit in float64).  The last test runs the pins against plausible mistakes
(a missing transpose, a dropped accumulation, a dropped UP factor) and checks
that each is caught.
"""
import types

import numpy as np
import pytest


def _ints(rng, shape):
    return rng.integers(-8, 9, size=shape).astype(np.float32)


def check_bwd_bruteforce_integers(orc, seed=10):
    rng = np.random.default_rng(seed)
    for (M, K, N) in [(1, 1, 1), (3, 4, 5), (5, 3, 2), (4, 4, 4), (7, 2, 6), (2, 8, 3)]:
        dY, W, X = _ints(rng, (M, N)), _ints(rng, (K, N)), _ints(rng, (M, K))
        Y0t, Y0a = _ints(rng, (M, K)), _ints(rng, (K, N))
        d, w, x = dY.astype(int).tolist(), W.astype(int).tolist(), X.astype(int).tolist()
        dx = [[sum(d[m][n] * w[k][n] for n in range(N)) for k in range(K)] for m in range(M)]
        dxb = [[sum(abs(d[m][n] * w[k][n]) for n in range(N)) for k in range(K)] for m in range(M)]
        dw = [[sum(x[m][k] * d[m][n] for m in range(M)) for n in range(N)] for k in range(K)]
        dwb = [[sum(abs(x[m][k] * d[m][n]) for m in range(M)) for n in range(N)] for k in range(K)]
        y, b = orc.matmul_t(dY, W, want_scale=True)
        assert np.array_equal(y, np.array(dx, float)) and np.array_equal(b, np.array(dxb, float)), (M, K, N)
        assert np.array_equal(orc.matmul_t(dY, W, Y0=Y0t), np.array(dx, float) + Y0t), (M, K, N)
        y, b = orc.matmul_at(X, dY, want_scale=True)
        assert np.array_equal(y, np.array(dw, float)) and np.array_equal(b, np.array(dwb, float)), (M, K, N)
        assert np.array_equal(orc.matmul_at(X, dY, Y0=Y0a), np.array(dw, float) + Y0a), (M, K, N)
        rows = np.array([K - 1, 0])
        assert np.array_equal(orc.matmul_at(X, dY, rows=rows), np.array(dw, float)[rows])


def check_bwd_adjoint(orc, seed=11):
    """<X W, dY> = <X, dY W^T> = <W, X^T dY>: a transposed or swapped operand
    anywhere breaks one of the two equalities."""
    rng = np.random.default_rng(seed)
    for (M, K, N) in [(6, 10, 7), (9, 4, 12), (8, 8, 8)]:
        X = rng.standard_normal((M, K), dtype=np.float32)
        W = rng.standard_normal((K, N), dtype=np.float32)
        dY = rng.standard_normal((M, N), dtype=np.float32)
        fwd = orc.gemm(X, W)
        lhs = float(np.sum(fwd * dY))
        mag = float(np.sum(np.abs(X.astype(float)) @ np.abs(W.astype(float)) * np.abs(dY)))
        t = float(np.sum(orc.matmul_t(dY, W) * X))
        a = float(np.sum(orc.matmul_at(X, dY) * W))
        assert abs(t - lhs) <= 1e-12 * mag and abs(a - lhs) <= 1e-12 * mag, (M, K, N)


def check_bwd_identity(orc, seed=12):
    rng = np.random.default_rng(seed)
    M, K = 7, 9
    dY = rng.standard_normal((M, K), dtype=np.float32)
    eye = np.eye(K, dtype=np.float32)
    assert np.array_equal(orc.matmul_t(dY, eye), dY.astype(float))          # W = I: dX = dY
    eyeM = np.eye(M, dtype=np.float32)
    assert np.array_equal(orc.matmul_at(eyeM, dY), dY.astype(float))        # X = I: dW = dY
    onehot = np.zeros((M, K), dtype=np.float32)
    onehot[2, 5] = 1.0
    want = np.zeros((K, K))
    want[5] = dY[2]
    assert np.array_equal(orc.matmul_at(onehot, dY), want)                  # row 5 of dW is row 2 of dY


def check_bwd_swiglu(orc, seed=13):
    from scipy.special import expit
    rng = np.random.default_rng(seed)
    M, K, N = 12, 9, 5
    G = rng.standard_normal((M, K), dtype=np.float32) * np.float32(4.0)
    G[0, :4] = [80.0, -80.0, 100.0, -1000.0]
    U = rng.standard_normal((M, K), dtype=np.float32)
    dY = rng.standard_normal((M, N), dtype=np.float32)
    Y0 = rng.standard_normal((K, N), dtype=np.float32)
    g, u = G.astype(float), U.astype(float)
    H = g * expit(g) * u
    ref = H.T @ dY.astype(float) + Y0
    scale = np.abs(H.T) @ np.abs(dY.astype(float))
    y, b = orc.matmul_at(G, dY, Y0=Y0, U=U, want_scale=True)
    assert np.all(np.abs(y - ref) <= 1e-13 * (scale + np.abs(Y0)))
    assert np.all(np.abs(b - scale) <= 1e-13 * scale)
    rows = np.array([3, 0, 8])
    assert np.array_equal(orc.matmul_at(G, dY, Y0=Y0, U=U, rows=rows), y[rows])


PINS = [check_bwd_bruteforce_integers, check_bwd_adjoint, check_bwd_identity, check_bwd_swiglu]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_pins(oracle_mod, pin):
    pin(oracle_mod)


def _mutant(orc, **overrides):
    ns = types.SimpleNamespace(gemm=orc.gemm, gemm_f64a=orc.gemm_f64a, a_operand=orc.a_operand,
                               matmul_t=orc.matmul_t, matmul_at=orc.matmul_at)
    for k, v in overrides.items():
        setattr(ns, k, v(orc))
    return ns


MUTANTS = {
    # the weight used without its transpose (square shapes only get that far)
    "t_no_transpose": {"matmul_t": lambda o: (lambda dY, W, Y0=None, rows=None, want_scale=False, threads=0:
                                              o.gemm(dY, np.ascontiguousarray(W), R=Y0, rows=rows,
                                                     want_scale=want_scale))},
    # the activation transposed the wrong way round: (dY^T X)^T of a square case
    "at_swapped": {"matmul_at": lambda o: (lambda X, dY, Y0=None, U=None, rows=None, want_scale=False, threads=0:
                                           o.gemm(np.ascontiguousarray(dY.T), X, R=Y0, rows=rows,
                                                  want_scale=want_scale))},
    # the _acc output's previous value ignored
    "t_acc_dropped": {"matmul_t": lambda o: (lambda dY, W, Y0=None, rows=None, want_scale=False, threads=0:
                                             o.matmul_t(dY, W, rows=rows, want_scale=want_scale))},
    # the UP factor of the SwiGLU activation dropped
    "at_swiglu_up_dropped": {"matmul_at": lambda o: (
        lambda X, dY, Y0=None, U=None, rows=None, want_scale=False, threads=0:
        o.matmul_at(X, dY, Y0=Y0, U=None if U is None else np.ones_like(U), rows=rows, want_scale=want_scale))},
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mistakes_are_caught(oracle_mod, name):
    mutant = _mutant(oracle_mod, **MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {name}"
