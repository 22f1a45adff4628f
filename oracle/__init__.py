"""Reference oracle for the forward linear-layer GEMM family (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, loads or calls it, and
the two share no source.

The arithmetic lives in ``oracle.cpp`` (plain C++, built by g++ with
``-ffp-contract=off``); this module only marshals numpy arrays into it and
implements the element-wise tolerance test.

Definition followed (pages of the llm.istanbul/learn series):

* "matmul ve matmul_residual — Tiled Matrix Multiply (Forward)", section
  "Ne Yapar?": Y = X @ W, Y = X @ W + R, Y = (silu(GATE) * UP) @ W + R; section
  "Önemli Optimizasyonlar" §1: f16 weights (vec4<f16>) staged into f32 tiles.
* "ffn_gelu_backward ve ffn_swiglu_backward — FFN Activation Backward",
  section "Türevler / SiLU'": silu(x) = x * sigmoid(x) with the sign-branched
  sigmoid.
* The backward linear family that "Ne Yapar?" names (matmul_t, matmul_at,
  their _acc forms and matmul_at_swiglu_a), read from the names:
  dX = dY @ W^T, dW = A^T @ dY with A = X or silu(GATE) * UP, and "_acc"
  adds the product to the output's previous value.  ``matmul_t`` and
  ``matmul_at`` are those definitions written out: an explicit transpose
  (a copy) followed by the pinned contraction ``gemm`` / ``gemm_f64a``.

Every exported function is pinned by ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

# Element-wise parity bounds |y - y_ref| <= rel * sum_k |a_ik||w_kj| + abs.
TOL_W32 = (2e-5, 1e-6)
TOL_W16 = (1e-3, 1e-5)

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (host only, no GPU code)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["g++", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c++17", "-shared", "-fPIC", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def configure(lib):
    """Declare the C signatures on a loaded liboracle handle."""
    p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.oracle_sigmoid.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_gemm_rows.argtypes = [p, p, p, c_int, p, i64, i64, i64, p, i64, p, p, c_int]
    lib.oracle_gemm_rows.restype = c_int
    lib.oracle_a_rows.argtypes = [p, p, i64, i64, p, i64, p]
    lib.oracle_a_rows.restype = c_int
    lib.oracle_gemm_rows_f64a.argtypes = [p, p, c_int, p, i64, i64, i64, p, c_int]
    lib.oracle_gemm_rows_f64a.restype = c_int
    lib.oracle_row_col_sums.argtypes = [p, p, p, c_int, p, i64, i64, i64, p, p, p, p, c_int]
    lib.oracle_row_col_sums.restype = c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a, name):
    if a is None:
        return None
    if a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous float32 array")
    return a


def half_to_double(bits: int) -> float:
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def sigmoid(x: float) -> float:
    return _load().oracle_sigmoid(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def gemm(A, W, R=None, U=None, rows=None, want_scale=False, threads=0):
    """Oracle forward GEMM on the given output rows.

    A: [M, K] float32 (X, or GATE when U is given); U: [M, K] float32 or None;
    W: [K, N] float32 or float16; R: [M, N] float32 or None.
    rows: None (all rows) or a 1-D int64 array of row indices.
    Returns y_ref [len(rows), N] float64, and the tolerance scale
    sum_k |a_ik||w_kj| of the same shape if want_scale.
    """
    A = _f32(A, "A")
    U = _f32(U, "U")
    R = _f32(R, "R")
    if W.dtype not in (np.float32, np.float16) or not W.flags.c_contiguous:
        raise TypeError("W must be a C-contiguous float32 or float16 array")
    M, K = A.shape
    K2, N = W.shape
    if K2 != K or (U is not None and U.shape != A.shape) or (R is not None and R.shape != (M, N)):
        raise ValueError("shape mismatch")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.shape[0]
    else:
        nrows = M
    y = np.empty((nrows, N), dtype=np.float64)
    b = np.empty((nrows, N), dtype=np.float64) if want_scale else None
    rc = _load().oracle_gemm_rows(_ptr(A), _ptr(U), _ptr(W), int(W.dtype == np.float16), _ptr(R),
                                  M, K, N, _ptr(rows), nrows, _ptr(y), _ptr(b), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows rejected its arguments (rc={rc})")
    return (y, b) if want_scale else y


def a_operand(A, U=None, rows=None):
    """The A operand as the contraction sees it (X, or silu(GATE)*UP), in double."""
    A = _f32(A, "A")
    U = _f32(U, "U")
    M, K = A.shape
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.shape[0]
    else:
        nrows = M
    h = np.empty((nrows, K), dtype=np.float64)
    rc = _load().oracle_a_rows(_ptr(A), _ptr(U), M, K, _ptr(rows), nrows, _ptr(h))
    if rc != 0:
        raise ValueError(f"oracle_a_rows rejected its arguments (rc={rc})")
    return h


def gemm_f64a(H, W, R=None, threads=0):
    """Oracle contraction with a float64 A operand (all rows)."""
    H = np.ascontiguousarray(H, dtype=np.float64)
    R = _f32(R, "R")
    M, K = H.shape
    N = W.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_rows_f64a(_ptr(H), _ptr(W), int(W.dtype == np.float16), _ptr(R),
                                       M, K, N, _ptr(y), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_rows_f64a rejected its arguments (rc={rc})")
    return y


def row_col_sums(A, W, R=None, U=None, threads=0):
    """Exact-in-fp64 row and column sums of the product and their magnitudes.

    Returns (row_sum [M], row_mag [M], col_sum [N], col_mag [N]) where
    row_sum[i] = sum_j y_ij, row_mag[i] = sum_j sum_k |a_ik||w_kj|, and the
    same over i for columns (R's sums are included in row_sum/col_sum).
    """
    A = _f32(A, "A")
    U = _f32(U, "U")
    R = _f32(R, "R")
    M, K = A.shape
    N = W.shape[1]
    rs, rm = np.empty(M), np.empty(M)
    cs, cm = np.empty(N), np.empty(N)
    rc = _load().oracle_row_col_sums(_ptr(A), _ptr(U), _ptr(W), int(W.dtype == np.float16), _ptr(R),
                                     M, K, N, _ptr(rs), _ptr(rm), _ptr(cs), _ptr(cm), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_row_col_sums rejected its arguments (rc={rc})")
    return rs, rm, cs, cm


def compare_sums(y, R, sums, tol):
    """Check the row and column sums of a result against row_col_sums().

    Each sum may differ by at most rel * (summed tolerance scale) + abs * count,
    plus 2^-23 * sum |y| for the rounding of the residual add and of y itself.
    Returns the worst ratio over all rows and columns and the failure count.
    """
    rel, ab = tol
    rs, rm, cs, cm = sums
    M, N = rs.shape[0], cs.shape[0]
    y_rows = np.zeros(M)
    y_rows_abs = np.zeros(M)
    y_cols = np.zeros(N)
    y_cols_abs = np.zeros(N)
    step = max(1, (1 << 24) // max(N, 1))
    for i0 in range(0, M, step):
        blk = np.asarray(y[i0:i0 + step], dtype=np.float64)
        y_rows[i0:i0 + step] = blk.sum(axis=1)
        y_rows_abs[i0:i0 + step] = np.abs(blk).sum(axis=1)
        y_cols += blk.sum(axis=0)
        y_cols_abs += np.abs(blk).sum(axis=0)
    r_bound = rel * rm + ab * N + 2.0 ** -23 * y_rows_abs
    c_bound = rel * cm + ab * M + 2.0 ** -23 * y_cols_abs
    with np.errstate(invalid="ignore"):
        r_ratio = np.abs(y_rows - rs) / r_bound
        c_ratio = np.abs(y_cols - cs) / c_bound
    r_ratio = np.where(np.isfinite(r_ratio), r_ratio, np.inf)
    c_ratio = np.where(np.isfinite(c_ratio), c_ratio, np.inf)
    worst = max(float(r_ratio.max(initial=0.0)), float(c_ratio.max(initial=0.0)))
    fails = int(np.count_nonzero(r_ratio > 1.0) + np.count_nonzero(c_ratio > 1.0))
    return {"max_ratio": worst, "fails": fails}


def compare(y, y_ref, scale, tol):
    """Element-wise parity test |y - y_ref| <= rel * scale + abs.

    y: float32 result; y_ref, scale: float64 from gemm(); tol: (rel, abs).
    A non-finite y where y_ref is finite fails.  Returns a dict with the worst
    error/bound ratio, the failure count and the worst (row, col).
    """
    rel, ab = tol
    y64 = np.asarray(y, dtype=np.float64)
    if y64.shape != y_ref.shape:
        raise ValueError(f"shape mismatch {y64.shape} vs {y_ref.shape}")
    bound = rel * scale + ab
    with np.errstate(invalid="ignore"):
        err = np.abs(y64 - y_ref)
        ratio = err / bound
    finite_both = np.isfinite(y64) & np.isfinite(y_ref)
    # Non-finite values pass only where both sides agree exactly (same
    # infinity, or NaN on both sides).
    same_special = (~finite_both) & ((y64 == y_ref) | (np.isnan(y64) & np.isnan(y_ref)))
    ratio = np.where(finite_both, ratio, np.where(same_special, 0.0, np.inf))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    fails = int(np.count_nonzero(ratio > 1.0))
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else (0, 0)
    return {
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "fails": fails,
        "worst": tuple(int(v) for v in worst),
        "n": int(ratio.size),
    }


def matmul_t(dY, W, Y0=None, rows=None, want_scale=False, threads=0):
    """matmul_t (Y0 None) or matmul_t_acc: dX = dY @ W^T (+ Y0).

    dY [M, N] float32, W [K, N] float32 (the forward's weight), Y0 [M, K]
    float32 or None.  Returns dX [len(rows), K] float64 (and the scale
    sum_n |dy_mn||w_kn| if want_scale), as gemm() does.
    """
    W = _f32(W, "W")
    Wt = np.ascontiguousarray(W.T)          # [N, K]: the transposed weight
    return gemm(dY, Wt, R=Y0, rows=rows, want_scale=want_scale, threads=threads)


def matmul_at(X, dY, Y0=None, U=None, rows=None, want_scale=False, threads=0):
    """matmul_at / matmul_at_acc / matmul_at_swiglu_a / matmul_at_acc_swiglu_a:
    dW = A^T @ dY (+ Y0), A = X, or silu(X) * U when U is given (X = GATE).

    X (and U) [M, K] float32, dY [M, N] float32, Y0 [K, N] float32 or None.
    rows: None or output rows (indices into K).  Returns dW [len(rows), N]
    float64 (and the scale sum_m |a_mk||dy_mn| if want_scale).
    """
    X = _f32(X, "X")
    dY = _f32(dY, "dY")
    Y0 = _f32(Y0, "Y0")
    if U is None:
        At = np.ascontiguousarray(X.T)      # [K, M]
        return gemm(At, dY, R=Y0, rows=rows, want_scale=want_scale, threads=threads)
    H = a_operand(X, U)                     # [M, K] float64, the combine in double
    Ht = np.ascontiguousarray(H.T)
    idx = np.arange(Ht.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    Ht = np.ascontiguousarray(Ht[idx])
    R = None if Y0 is None else np.ascontiguousarray(Y0[idx])
    y = gemm_f64a(Ht, dY, R=R, threads=threads)
    if not want_scale:
        return y
    b = gemm_f64a(np.abs(Ht), np.ascontiguousarray(np.abs(dY)), threads=threads)
    return y, b
