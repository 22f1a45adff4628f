"""Pins for the fp64 CPU oracle, against values fixed by something other than
the oracle itself: IEEE 754 binary16 encodings worked by hand, exact rational
arithmetic on small inputs, closed forms of the sigmoid, scipy's expit, a
50-digit Decimal evaluation, numpy's float64 matmul, and special weight
matrices (identity, one-hot, zero) whose product is known exactly.

The last group plants mistakes into copies of the oracle source (built on the
CPU) and checks that the pins catch each one.
"""
import ctypes
import math
import os
import subprocess
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from tiled_dense_gemm_matmul_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# pin bodies (plain functions so the planted-mistake tests can rerun them)
# --------------------------------------------------------------------------

def _golden_binary16():
    rows = []
    with open(os.path.join(GOLDEN, "binary16_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            bits, val = line.split()[:2]
            rows.append((int(bits, 16), float(val)))
    return rows


def check_binary16_golden(orc):
    for bits, val in _golden_binary16():
        got = orc.half_to_double(bits)
        if math.isnan(val):
            assert math.isnan(got), hex(bits)
        else:
            assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), (hex(bits), got, val)


def check_binary16_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_sigmoid_closed_forms(orc):
    assert orc.sigmoid(0.0) == 0.5
    assert orc.silu(0.0) == 0.0
    for x in [1e-30, 1e-8, 0.1, 0.5, 1.0, 2.5, 7.0, 20.0, 36.0, 80.0, 100.0, 700.0]:
        s, t = orc.sigmoid(x), orc.sigmoid(-x)
        assert abs((s + t) - 1.0) <= 2.3e-16, x
        assert s >= 0.5 >= t
        # silu(x) - silu(-x) = x * (sigma(x) + sigma(-x)) = x
        assert abs(orc.silu(x) - orc.silu(-x) - x) <= 4.5e-16 * abs(x), x
    # the branch keeps exp() from overflowing: no NaN / Inf far out
    assert orc.sigmoid(1000.0) == 1.0
    assert orc.sigmoid(-1000.0) == 0.0
    assert orc.silu(-1000.0) == 0.0 and not math.copysign(1.0, orc.silu(-1000.0)) > 0
    assert orc.silu(1000.0) == 1000.0
    assert orc.sigmoid(-745.0) > 0.0  # exp(-745) is the smallest double subnormal
    assert math.isnan(orc.sigmoid(float("nan")))


def check_sigmoid_expit(orc):
    from scipy.special import expit
    xs = np.concatenate([np.linspace(-40, 40, 801), [-745.0, -700.0, -100.0, -80.0, -88.7, 80.0, 88.7, 100.0, 700.0, 745.0]])
    for x in xs:
        ref = float(expit(x))
        got = orc.sigmoid(float(x))
        assert abs(got - ref) <= 4e-16 * abs(ref) + 1e-300, (x, got, ref)


def check_sigmoid_decimal(orc):
    getcontext().prec = 60
    for x in [-80.0, -30.0, -10.0, -3.0, -1.0, -0.25, 0.25, 1.0, 3.0, 10.0, 30.0, 80.0, math.log(3.0)]:
        d = Decimal(x)
        ref = Decimal(1) / (Decimal(1) + (-d).exp())
        got = Decimal(orc.sigmoid(x))
        assert abs(got - ref) <= Decimal("3e-16") * ref, x
        sref = d * ref
        sgot = Decimal(orc.silu(x))
        assert abs(sgot - sref) <= Decimal("5e-16") * abs(sref), x


def _parse_mat(text):
    return [[int(v) for v in row.split(",")] for row in text.split(";")]


def check_hand_example(orc):
    vals = {}
    with open(os.path.join(GOLDEN, "matmul_hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split("=", 1)
            vals[key.strip()] = _parse_mat(rhs)
    X = np.array(vals["X"], dtype=np.float32)
    W = np.array(vals["W"], dtype=np.float32)
    R = np.array(vals["R"], dtype=np.float32)
    UP = np.array(vals["UP"], dtype=np.float32)
    assert np.array_equal(orc.gemm(X, W), np.array(vals["XW"], dtype=np.float64))
    assert np.array_equal(orc.gemm(X, W, R=R), np.array(vals["XW_plus_R"], dtype=np.float64))
    G0 = np.zeros_like(UP)
    assert np.array_equal(orc.gemm(G0, W, R=R, U=UP), np.array(vals["SWIGLU_GATE0"], dtype=np.float64))
    # f16 weights holding the same small integers decode exactly
    assert np.array_equal(orc.gemm(X, W.astype(np.float16), R=R), np.array(vals["XW_plus_R"], dtype=np.float64))


def check_bruteforce_integers(orc, seed=0):
    rng = np.random.default_rng(seed)
    dims = [1, 2, 3, 4, 5, 7, 8]
    for M in dims:
        for K in dims:
            for N in dims:
                X = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
                W = rng.integers(-8, 9, size=(K, N)).astype(np.float32)
                R = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
                xi, wi, ri = X.astype(int).tolist(), W.astype(int).tolist(), R.astype(int).tolist()
                exact = [[sum(xi[i][k] * wi[k][j] for k in range(K)) for j in range(N)] for i in range(M)]
                exact_b = [[sum(abs(xi[i][k] * wi[k][j]) for k in range(K)) for j in range(N)] for i in range(M)]
                y, b = orc.gemm(X, W, want_scale=True)
                assert np.array_equal(y, np.array(exact, dtype=np.float64)), (M, K, N)
                assert np.array_equal(b, np.array(exact_b, dtype=np.float64)), (M, K, N)
                exact_r = [[exact[i][j] + ri[i][j] for j in range(N)] for i in range(M)]
                assert np.array_equal(orc.gemm(X, W, R=R), np.array(exact_r, dtype=np.float64))
                assert np.array_equal(orc.gemm(X, W.astype(np.float16), R=R), np.array(exact_r, dtype=np.float64))


def check_bruteforce_rational(orc, seed=1):
    """Random fp32 X against random f16 W (subnormals included), checked
    against exact rational arithmetic: the fp64 sum may only differ by the
    rounding of K additions."""
    rng = np.random.default_rng(seed)
    for (M, K, N) in [(3, 5, 4), (4, 8, 3), (2, 16, 5), (5, 7, 7)]:
        X = rng.standard_normal((M, K), dtype=np.float32)
        bits = rng.integers(0, 0x7C00, size=(K, N), dtype=np.uint16)  # finite magnitudes
        bits |= (rng.integers(0, 2, size=(K, N)).astype(np.uint16) << 15)
        W = bits.view(np.float16)
        R = rng.standard_normal((M, N), dtype=np.float32)
        y, b = orc.gemm(X, W, R=R, want_scale=True)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(X[i, k])) * Fraction(float(W[k, j])) for k in range(K)]
                exact = sum(terms, Fraction(0)) + Fraction(float(R[i, j]))
                mag = sum((abs(t) for t in terms), Fraction(0))
                bound = (K + 1) * 2.0 ** -52 * (float(mag) + abs(float(R[i, j])))
                assert abs(Fraction(y[i, j]) - exact) <= Fraction(bound), (M, K, N, i, j)
                assert abs(Fraction(b[i, j]) - mag) <= Fraction(K * 2.0 ** -52 * float(mag)), (i, j)


def check_special_weights(orc, seed=2):
    rng = np.random.default_rng(seed)
    M, K = 9, 12
    X = rng.standard_normal((M, K), dtype=np.float32)
    R = rng.standard_normal((M, K), dtype=np.float32)
    eye = np.eye(K, dtype=np.float32)
    assert np.array_equal(orc.gemm(X, eye), X.astype(np.float64))
    assert np.array_equal(orc.gemm(X, eye.astype(np.float16)), X.astype(np.float64))
    assert np.array_equal(orc.gemm(X, eye, R=R), X.astype(np.float64) + R.astype(np.float64))
    N = 7
    R2 = rng.standard_normal((M, N), dtype=np.float32)
    for (k0, j0) in [(0, 0), (K - 1, N - 1), (5, 2)]:
        onehot = np.zeros((K, N), dtype=np.float32)
        onehot[k0, j0] = 1.0
        y = orc.gemm(X, onehot)
        want = np.zeros((M, N))
        want[:, j0] = X[:, k0]
        assert np.array_equal(y, want), (k0, j0)
        y = orc.gemm(X, onehot, R=R2)
        want = R2.astype(np.float64).copy()
        want[:, j0] += X[:, k0].astype(np.float64)
        assert np.array_equal(y, want), (k0, j0)
    zero = np.zeros((K, N), dtype=np.float32)
    assert np.array_equal(orc.gemm(X, zero, R=R2), R2.astype(np.float64))
    G = rng.standard_normal((M, K), dtype=np.float32)
    assert np.array_equal(orc.gemm(G, zero, R=R2, U=X), R2.astype(np.float64))


def check_swiglu(orc, seed=3):
    from scipy.special import expit
    rng = np.random.default_rng(seed)
    M, K, N = 6, 40, 5
    G = rng.standard_normal((M, K), dtype=np.float32) * np.float32(4.0)
    G[0, :6] = [80.0, -80.0, 100.0, -100.0, 1000.0, -1000.0]
    U = rng.standard_normal((M, K), dtype=np.float32)
    W = (rng.standard_normal((K, N), dtype=np.float32) * np.float32(0.02))
    R = rng.standard_normal((M, N), dtype=np.float32)
    H = orc.a_operand(G, U)
    g64, u64 = G.astype(np.float64), U.astype(np.float64)
    H_np = g64 * expit(g64) * u64
    assert np.allclose(H, H_np, rtol=1e-15, atol=1e-300)
    assert H[0, 4] == 1000.0 * float(U[0, 4]) and H[0, 5] == 0.0
    # identity, bit for bit: swiglu_a(G, U, W, R) == matmul_residual(silu(G)*U, W, R)
    y_sw = orc.gemm(G, W, R=R, U=U)
    assert np.array_equal(y_sw, orc.gemm_f64a(H, W, R=R))
    # and against numpy's float64 product of the independently formed H
    y_np = H_np @ W.astype(np.float64) + R.astype(np.float64)
    scale = np.abs(H_np) @ np.abs(W.astype(np.float64)) + np.abs(R)
    assert np.all(np.abs(y_sw - y_np) <= 1e-13 * scale)
    # the identity-W probe used on the GPU side: Y = silu(G) * U + R
    Wi = np.eye(K, dtype=np.float32)
    Ri = rng.standard_normal((M, K), dtype=np.float32)
    assert np.array_equal(orc.gemm(G, Wi, R=Ri, U=U), H + Ri.astype(np.float64))


def check_numpy_crosscheck(orc):
    for case in (inputs.cfg1(), inputs.cfg2()):
        X, W = case["X"], case["W"]
        R = case.get("R")
        y, b = orc.gemm(X, W, R=R, want_scale=True)
        ref = X.astype(np.float64) @ W.astype(np.float64)
        bref = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64))
        if R is not None:
            ref = ref + R.astype(np.float64)
        assert np.all(np.abs(y - ref) <= 1e-12 * (b + (np.abs(R) if R is not None else 0)))
        assert np.all(np.abs(b - bref) <= 1e-12 * bref)


# --------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------

def test_binary16_golden(oracle_mod):
    check_binary16_golden(oracle_mod)


def test_binary16_exhaustive(oracle_mod):
    check_binary16_exhaustive(oracle_mod)


def test_sigmoid_closed_forms(oracle_mod):
    check_sigmoid_closed_forms(oracle_mod)


def test_sigmoid_vs_expit(oracle_mod):
    check_sigmoid_expit(oracle_mod)


def test_sigmoid_vs_decimal(oracle_mod):
    check_sigmoid_decimal(oracle_mod)


def test_hand_example(oracle_mod):
    check_hand_example(oracle_mod)


def test_bruteforce_integers(oracle_mod):
    check_bruteforce_integers(oracle_mod)


def test_bruteforce_rational(oracle_mod):
    check_bruteforce_rational(oracle_mod)


def test_special_weights(oracle_mod):
    check_special_weights(oracle_mod)


def test_swiglu(oracle_mod):
    check_swiglu(oracle_mod)


def test_numpy_crosscheck(oracle_mod):
    check_numpy_crosscheck(oracle_mod)


def test_row_subset_matches_full(oracle_mod):
    case = inputs.random_case(11, 37, 24, 20, swiglu=True, w16=True, residual=True)
    y, b = oracle_mod.gemm(case["G"], case["W"], R=case["R"], U=case["U"], want_scale=True)
    rows = np.array([36, 0, 17, 17, 5])
    ys, bs = oracle_mod.gemm(case["G"], case["W"], R=case["R"], U=case["U"], rows=rows, want_scale=True)
    assert np.array_equal(ys, y[rows]) and np.array_equal(bs, b[rows])


def test_degenerate_shapes(oracle_mod):
    X = np.zeros((3, 0), dtype=np.float32)
    W = np.zeros((0, 4), dtype=np.float32)
    R = np.arange(12, dtype=np.float32).reshape(3, 4)
    assert np.array_equal(oracle_mod.gemm(X, W), np.zeros((3, 4)))
    assert np.array_equal(oracle_mod.gemm(X, W, R=R), R.astype(np.float64))
    assert oracle_mod.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 4), np.float32)).shape == (0, 4)


def test_compare_semantics(oracle_mod):
    yref = np.array([[1.0, 2.0, np.inf, np.nan]])
    scale = np.ones_like(yref)
    ok = oracle_mod.compare(np.array([[1.0, 2.0, np.inf, np.nan]], np.float32), yref, scale, (1e-3, 0))
    assert ok["fails"] == 0
    bad = oracle_mod.compare(np.array([[1.01, np.nan, -np.inf, 0.0]], np.float32), yref, scale, (1e-3, 0))
    assert bad["fails"] == 4


def test_tolerance_discriminates(oracle_mod):
    """The fp32-W bound accepts true fp32 arithmetic in any summation order
    but rejects operands rounded to a 10-bit mantissa (TF32-style)."""
    case = inputs.cfg3()
    rows = np.arange(0, 512, 8)
    G, U, W, R = case["G"][rows], case["U"][rows], case["W"], case["R"][rows]
    y_ref, b = oracle_mod.gemm(G, W, R=R, U=U, want_scale=True)
    g = G.astype(np.float32)
    s = np.where(g >= 0, 1 / (1 + np.exp(-np.abs(g))), np.exp(-np.abs(g)) / (1 + np.exp(-np.abs(g)))).astype(np.float32)
    H32 = (g * s * U).astype(np.float32)
    y32 = (H32 @ W + R).astype(np.float32)
    assert oracle_mod.compare(y32, y_ref, b, oracle_mod.TOL_W32)["fails"] == 0
    acc = np.zeros((len(rows), W.shape[1]), np.float32)
    for k in range(W.shape[0]):  # sequential k-ascending fp32 chain
        acc += H32[:, k:k + 1] * W[k:k + 1, :]
    assert oracle_mod.compare(acc + R, y_ref, b, oracle_mod.TOL_W32)["fails"] == 0

    def tf32(a):
        bits = a.astype(np.float32).view(np.uint32)
        bits = (bits + np.uint32(0x1000)) & np.uint32(0xFFFFE000)
        return bits.view(np.float32)
    y_tf = (tf32(H32).astype(np.float64) @ tf32(W).astype(np.float64) + R).astype(np.float32)
    assert oracle_mod.compare(y_tf, y_ref, b, oracle_mod.TOL_W32)["fails"] > 0


# --------------------------------------------------------------------------
# planted mistakes: each mutated copy of oracle.cpp must fail some pin
# --------------------------------------------------------------------------

MUTATIONS = [
    ("sigmoid_sign", "return 1.0 / (1.0 + std::exp(-x));", "return 1.0 / (1.0 + std::exp(x));",
     [check_sigmoid_closed_forms, check_sigmoid_expit]),
    ("sigmoid_neg_branch", "return e / (1.0 + e);", "return 1.0 / (1.0 + e);",
     [check_sigmoid_expit, check_swiglu]),
    ("silu_dropped_x", "double oracle_silu(double x) { return x * oracle_sigmoid(x); }",
     "double oracle_silu(double x) { return oracle_sigmoid(x); }", [check_swiglu]),
    ("swiglu_dropped_up", "return oracle_silu(static_cast<double>(A[idx])) * static_cast<double>(U[idx]);",
     "return oracle_silu(static_cast<double>(A[idx]));", [check_swiglu]),
    ("residual_dropped", "yrow[j] = R ? acc[j] + static_cast<double>(R[i * N + j]) : acc[j];",
     "yrow[j] = acc[j];", [check_bruteforce_integers, check_hand_example]),
    ("k_reversed_on_a", "const double aik = a[k];", "const double aik = a[K - 1 - k];",
     [check_bruteforce_integers]),
    ("half_bias", "expo - 25", "expo - 24", [check_binary16_golden, check_binary16_exhaustive]),
    ("half_subnormal", "static_cast<double>(frac), -24", "static_cast<double>(frac), -25",
     [check_binary16_golden, check_binary16_exhaustive]),
    ("half_sign_dropped", "return sign ? -mag : mag;", "return mag;",
     [check_binary16_golden, check_bruteforce_rational]),
    ("scale_signed", "const double aik = std::fabs(a[k]);", "const double aik = a[k];",
     [check_bruteforce_integers]),
    ("rowsum_dropped_residual", "if (row_sum) row_sum[i] = s + rs;", "if (row_sum) row_sum[i] = s;",
     [lambda o: check_row_col_sums(o)]),
    ("colsum_wrong_weight", "s += asum[k] * w;", "s += aabs[k] * w;", [lambda o: check_row_col_sums(o)]),
]


class _MutantOracle:
    """The oracle's Python surface bound to a mutated library."""

    def __init__(self, orc, lib):
        self._orc, self._lib = orc, lib

    def __getattr__(self, name):
        orc, lib = self._orc, self._lib
        fn = getattr(orc, name)
        if not callable(fn):
            return fn

        def wrapped(*a, **k):
            saved = orc._lib
            orc._lib = lib
            try:
                return fn(*a, **k)
            finally:
                orc._lib = saved
        return wrapped


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(oracle_mod, tmp_path, name, old, new, pins):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "oracle.cpp")).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    cpp = tmp_path / f"{name}.cpp"
    so = tmp_path / f"{name}.so"
    cpp.write_text(mutated)
    subprocess.run(["g++", "-O1", "-fopenmp", "-ffp-contract=off", "-std=c++17", "-shared", "-fPIC",
                    str(cpp), "-o", str(so)], check=True)
    mutant = _MutantOracle(oracle_mod, oracle_mod.configure(ctypes.CDLL(str(so))))
    caught = []
    for pin in pins:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(getattr(pin, "__name__", "pin"))
    assert caught, f"no pin caught planted mistake {name}"


def check_row_col_sums(orc, seed=4):
    for (M, K, N, sw, w16, res) in [(7, 12, 9, False, False, True), (5, 20, 8, True, True, True),
                                      (6, 8, 4, False, True, False)]:
        case = inputs.random_case(seed, M, K, N, swiglu=sw, w16=w16, residual=res)
        A = case["G"] if sw else case["X"]
        U = case.get("U")
        R = case.get("R")
        y, b = orc.gemm(A, case["W"], R=R, U=U, want_scale=True)
        rs, rm, cs, cm = orc.row_col_sums(A, case["W"], R=R, U=U)
        tot = np.abs(y).sum() + b.sum() + 1.0
        assert np.allclose(rs, y.sum(axis=1), rtol=0, atol=1e-13 * tot)
        assert np.allclose(cs, y.sum(axis=0), rtol=0, atol=1e-13 * tot)
        assert np.allclose(rm, b.sum(axis=1), rtol=1e-13)
        assert np.allclose(cm, b.sum(axis=0), rtol=1e-13)
        # integers: exact
    case = inputs.random_case(seed, 6, 16, 10, integer=True, residual=True)
    X, W, R = case["X"], case["W"], case["R"]
    rs, rm, cs, cm = orc.row_col_sums(X, W, R=R)
    Xi, Wi, Ri = X.astype(np.int64), W.astype(np.int64), R.astype(np.int64)
    Yi = Xi @ Wi + Ri
    assert np.array_equal(rs, Yi.sum(axis=1).astype(np.float64))
    assert np.array_equal(cs, Yi.sum(axis=0).astype(np.float64))
    assert np.array_equal(rm, (np.abs(Xi) @ np.abs(Wi)).sum(axis=1).astype(np.float64))


def test_row_col_sums(oracle_mod):
    check_row_col_sums(oracle_mod)


def test_compare_sums_detects_a_wrong_row(oracle_mod):
    case = inputs.random_case(9, 40, 64, 24, residual=True)
    y = oracle_mod.gemm(case["X"], case["W"], R=case["R"]).astype(np.float32)
    sums = oracle_mod.row_col_sums(case["X"], case["W"], R=case["R"])
    assert oracle_mod.compare_sums(y, case["R"], sums, oracle_mod.TOL_W32)["fails"] == 0
    y_bad = y.copy()
    y_bad[13, 5] += 0.01
    assert oracle_mod.compare_sums(y_bad, case["R"], sums, oracle_mod.TOL_W32)["fails"] >= 2
