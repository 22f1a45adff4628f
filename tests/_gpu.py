"""Shared plumbing for the GPU tests: move seeded host arrays to the device,
run the library through its binding, and check against the oracle."""
import sys

import numpy as np

import oracle

DEV = None


def device():
    global DEV
    import torch
    if DEV is None:
        if not torch.cuda.is_available():
            raise RuntimeError("GPU tests need a HIP device (cuda:0)")
        DEV = torch.device("cuda:0")
    return DEV


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def run(case, config=None, out=None):
    """Run the case's variant on the GPU; returns the device output tensor."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    W = to_dev(case["W"])
    R = to_dev(case["R"]) if case.get("R") is not None else None
    if "G" in case:
        y = binding.matmul_residual_swiglu_a(to_dev(case["G"]), to_dev(case["U"]), W, R, out=out, config=config)
    else:
        y = binding.matmul(to_dev(case["X"]), W, R, out=out, config=config)
    torch.cuda.synchronize()
    return y


def tol_for(case):
    return oracle.TOL_W16 if case["W"].dtype == np.float16 else oracle.TOL_W32


def oracle_ref(case, rows=None, want_scale=True):
    A = case["G"] if "G" in case else case["X"]
    return oracle.gemm(A, case["W"], R=case.get("R"), U=case.get("U"), rows=rows, want_scale=want_scale)


def check(case, y, rows=None, label=""):
    """Element-wise parity of y (host float32, the selected rows) against the oracle."""
    y_ref, b = oracle_ref(case, rows=rows)
    res = oracle.compare(y, y_ref, b, tol_for(case))
    say(f"  {label}: max err/tol = {res['max_ratio']:.4g}, fails = {res['fails']} of {res['n']}, worst {res['worst']}")
    assert res["fails"] == 0, res
    return res


def check_sums(case, y, label=""):
    A = case["G"] if "G" in case else case["X"]
    sums = oracle.row_col_sums(A, case["W"], R=case.get("R"), U=case.get("U"))
    res = oracle.compare_sums(y, case.get("R"), sums, tol_for(case))
    say(f"  {label}: row/col sums max err/tol = {res['max_ratio']:.4g}, fails = {res['fails']}")
    assert res["fails"] == 0, res
    return res
