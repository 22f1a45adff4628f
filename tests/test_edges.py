"""Edge cases of the HIP path: ragged and tiny shapes, K = 0, exactness on
integer inputs (every configuration) and special weights, the sigmoid branch
far out, binary16 subnormal weights, run-to-run determinism, the error path
for an aliased output and the timing events.  The out-of-bounds guards are in
test_guards.py."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import check, device, run, say, to_dev

pytestmark = pytest.mark.gpu


def _lib():
    from tiled_dense_gemm_matmul_amd import binding
    return binding


@pytest.mark.parametrize("M", [1, 63, 65, 129])
@pytest.mark.parametrize("N", [4, 68, 132])
@pytest.mark.parametrize("K", [4, 20, 772])
def test_ragged_shapes(M, N, K):
    say(f"ragged M={M} K={K} N={N}")
    c = inputs.random_case(M + 1000 * N + K, M, K, N, residual=True)
    check(c, run(c).cpu().numpy(), label="matmul_residual")
    c = inputs.random_case(M + 1000 * N + K + 1, M, K, N, swiglu=True, w16=True, residual=True, gate_scale=3.0)
    check(c, run(c).cpu().numpy(), label="swiglu_w16")


@pytest.mark.parametrize("M,K,N", [(1, 4100, 4), (3, 2052, 4), (1, 8192, 48)])
def test_split_k_on_tiny_outputs(M, K, N):
    # one to three output rows over a long contraction: the library's
    # choice splits K (every form below but SwiGLU with fp32 W at these
    # lengths); each product with and without a workspace, every element
    # against the oracle
    import torch
    b = _lib()
    for sw, w16 in ((False, False), (True, False), (False, True), (True, True)):
        tile = b.kernel_config(M, K, N, swiglu=sw, w16=w16)
        say(f"tiny output {M}x{K}x{N} swiglu={sw} w16={w16} -> {tile}")
        assert "_ks" in tile or (sw and not w16)
        c = inputs.random_case(M + K + N + 2 * sw + w16, M, K, N, swiglu=sw, w16=w16, residual=sw, gate_scale=3.0)
        d = {k: to_dev(v) for k, v in c.items()}
        for ws in (True, False):
            if sw:
                y = b.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], use_workspace=ws)
            else:
                y = b.matmul(d["X"], d["W"], use_workspace=ws)
            torch.cuda.synchronize()
            check(c, y.cpu().numpy(), label=f"workspace={ws}")


@pytest.mark.parametrize("M,K,N", [(1, 4, 4100), (3, 8, 8196)])
def test_split_k_on_tiny_backward_outputs(M, K, N):
    # the backward products onto one to three rows (dX) or a 4 x 4 / 8 x 4
    # block (dW) over a long contraction: K split with a workspace, not
    # without; every element against the oracle
    import torch
    b = _lib()
    assert "_ks" in b.bwd_kernel_config("matmul_t", M, K, N)
    c = inputs.backward_case(M + K + N, M, K, N)
    for ws in (True, False):
        y = b.matmul_t(to_dev(c["dY"]), to_dev(c["W"]), use_workspace=ws)
        torch.cuda.synchronize()
        ref, scale = oracle.matmul_t(c["dY"], c["W"], want_scale=True)
        res = oracle.compare(y.cpu().numpy(), ref, scale, oracle.TOL_W32)
        say(f"  matmul_t {M}x{K}x{N} workspace={ws}: max err/tol {res['max_ratio']:.3g}")
        assert res["fails"] == 0, res
    # dW [K2 x N2] over N tokens
    T, K2, N2 = N, K, 4
    assert "_ks" in b.bwd_kernel_config("matmul_at", T, K2, N2)
    c = inputs.backward_case(T + K2, T, K2, N2, swiglu=True, gate_scale=3.0)
    for sw in (False, True):
        for ws in (True, False):
            if sw:
                y = b.matmul_at_swiglu_a(to_dev(c["G"]), to_dev(c["U"]), to_dev(c["dY"]), use_workspace=ws)
            else:
                y = b.matmul_at(to_dev(c["G"]), to_dev(c["dY"]), use_workspace=ws)
            torch.cuda.synchronize()
            ref, scale = oracle.matmul_at(c["G"], c["dY"], U=c["U"] if sw else None, want_scale=True)
            res = oracle.compare(y.cpu().numpy(), ref, scale, oracle.TOL_W32)
            say(f"  matmul_at{'_swiglu_a' if sw else ''} {T}x{K2}x{N2} workspace={ws}: max err/tol {res['max_ratio']:.3g}")
            assert res["fails"] == 0, res


def test_k_zero():
    import torch
    b = _lib()
    R = to_dev(np.arange(12, dtype=np.float32).reshape(3, 4))
    X = torch.zeros((3, 0), dtype=torch.float32, device=device())
    W = torch.zeros((0, 4), dtype=torch.float32, device=device())
    y = b.matmul(X, W, R)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), R.cpu())
    y = b.matmul(X, W)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), torch.zeros(3, 4))


def test_empty_outputs():
    import torch
    b = _lib()
    X = torch.zeros((0, 8), dtype=torch.float32, device=device())
    W = torch.zeros((8, 4), dtype=torch.float32, device=device())
    assert b.matmul(X, W).shape == (0, 4)
    X = torch.zeros((5, 8), dtype=torch.float32, device=device())
    W = torch.zeros((8, 0), dtype=torch.float32, device=device())
    assert b.matmul(X, W).shape == (5, 0)


@pytest.mark.parametrize("cfg", [None] + list(range(40)))
def test_integer_inputs_bit_exact(cfg):
    b = _lib()
    if cfg is not None and cfg >= b.num_configs():
        pytest.skip("no such config")
    for (M, K, N) in [(96, 3072, 64), (257, 768, 260)]:
        for w16 in (False, True):
            if w16 and cfg is not None and not b.config_takes_w16(cfg):
                continue  # fp32-only tile (W in registers)
            c = inputs.random_case(M + K, M, K, N, w16=w16, residual=True, integer=True)
            say(f"integer M={M} K={K} N={N} w16={w16} config={cfg}")
            y = run(c, config=cfg).cpu().numpy()
            y_ref = oracle.gemm(c["X"], c["W"], R=c["R"])
            assert np.array_equal(y.astype(np.float64), y_ref)


def test_zero_and_identity_weights_bitwise():
    M, K = 130, 196
    rng = np.random.default_rng(5)
    X = rng.standard_normal((M, K), dtype=np.float32)
    R = rng.standard_normal((M, K), dtype=np.float32)
    zero = {"X": X, "W": np.zeros((K, K), np.float32), "R": R}
    assert np.array_equal(run(zero).cpu().numpy(), R)
    eye = {"X": X, "W": np.eye(K, dtype=np.float32)}
    assert np.array_equal(run(eye).cpu().numpy(), X)
    eye16 = {"X": X, "W": np.eye(K, dtype=np.float16)}
    assert np.array_equal(run(eye16).cpu().numpy(), X)
    G = rng.standard_normal((M, K), dtype=np.float32)
    sw0 = {"G": G, "U": X, "W": np.zeros((K, K), np.float32), "R": R}
    assert np.array_equal(run(sw0).cpu().numpy(), R)


def test_silu_probe_far_out():
    """Identity W makes Y = silu(G) * U + R: the sigmoid's two branches at
    +-80, +-100, +-1000, zero and tiny gates, against the oracle."""
    K = 64
    vals = np.array([80, -80, 100, -100, 1000, -1000, 0.0, -0.0, 1e-30, -1e-30, 88.0, -88.0, 89.0, -89.0,
                     20, -20, 5, -5, 1, -1, 0.5, -0.5, 1e-3, -1e-3], dtype=np.float32)
    M = 8
    G = np.resize(vals, (M, K)).astype(np.float32)
    rng = np.random.default_rng(6)
    U = rng.standard_normal((M, K), dtype=np.float32)
    R = rng.standard_normal((M, K), dtype=np.float32)
    c = {"G": G, "U": U, "W": np.eye(K, dtype=np.float32), "R": R}
    y = run(c).cpu().numpy()
    assert np.all(np.isfinite(y))
    h = oracle.a_operand(G, U)
    # a handful of fp32 roundings: the exponential, the reciprocal, two products, the add
    err = np.abs(y.astype(np.float64) - (h + R.astype(np.float64)))
    assert np.all(err <= 8 * 2.0 ** -24 * (np.abs(h) + np.abs(R)) + 1e-37), float(err.max())
    check(c, y, label="silu probe")


def test_f16_subnormal_weights_are_not_flushed():
    M, K, N = 64, 64, 64
    rng = np.random.default_rng(8)
    X = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    bits = np.zeros((K, N), np.uint16)
    for j in range(N):
        bits[(j * 7) % K, j] = 1 + j * 16      # subnormal binary16 (exponent field 0)
        bits[(j * 3 + 1) % K, j] = 0x8000 | (3 + j)
    W = bits.view(np.float16)
    assert np.all(np.abs(W.astype(np.float32)) < 2.0 ** -14)
    c = {"X": X, "W": W}
    y = run(c).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), oracle.gemm(X, W))
    assert np.count_nonzero(y) > M * N // 2


def test_deterministic():
    c = inputs.cfg3()
    a = run(c).cpu().numpy()
    b = run(c).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_aliased_output_is_rejected():
    b = _lib()
    c = inputs.random_case(3, 64, 64, 64, residual=True)
    X, W, R = to_dev(c["X"]), to_dev(c["W"]), to_dev(c["R"])
    keep = R.clone()
    with pytest.raises(b.GemmError) as e:
        b.matmul(X, W, R, out=R)
    assert e.value.status == -5
    import torch
    torch.cuda.synchronize()
    assert torch.equal(R, keep)


@pytest.mark.parametrize("swiglu", [False, True])
def test_event_options_match_and_record(swiglu):
    """gemm_fwd_ex / gemm_fwd_swiglu_ex with start and stop events compute
    exactly what the plain entry points compute and leave a positive kernel
    time in the caller's events."""
    import torch
    b = _lib()
    lib = b.load_library()
    c = inputs.random_case(11, 200, 320, 136, swiglu=swiglu, w16=swiglu, residual=True)
    say(f"event options swiglu={swiglu} M=200 K=320 N=136")
    W, R = to_dev(c["W"]), to_dev(c["R"])
    M, K, N = 200, 320, 136
    y0 = torch.empty((M, N), device=device())
    y1 = torch.full((M, N), float("nan"), device=device())
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    e1.record(st)
    o = b.opts(-1, None, 0, e0.cuda_event, e1.cuda_event)
    if swiglu:
        G, U = to_dev(c["G"]), to_dev(c["U"])
        a = (G.data_ptr(), U.data_ptr(), W.data_ptr(), R.data_ptr())
        assert lib.gemm_fwd_swiglu(*a, y0.data_ptr(), M, K, N, 1, st.cuda_stream) == 0
        assert lib.gemm_fwd_swiglu_ex(*a, y1.data_ptr(), M, K, N, 1, o, st.cuda_stream) == 0
    else:
        X = to_dev(c["X"])
        a = (X.data_ptr(), W.data_ptr(), R.data_ptr())
        assert lib.gemm_fwd(*a, y0.data_ptr(), M, K, N, 0, st.cuda_stream) == 0
        assert lib.gemm_fwd_ex(*a, y1.data_ptr(), M, K, N, 0, o, st.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    assert e0.elapsed_time(e1) > 0.0
    check(c, y1.cpu().numpy(), label="events")


def test_timing_events():
    """The library's timing events (no system-scope fence when recorded):
    recorded by a launch at the kernel's start and end, they give a positive
    time no longer than a torch event pair around the same launch; recorded
    as markers around a launch, a positive time; the results are those of
    the plain entry point; NULL arguments are refused."""
    import ctypes

    import torch
    b = _lib()
    lib = b.load_library()
    M, K, N = 512, 768, 768
    c = inputs.random_case(12, M, K, N, residual=True)
    X, W, R = to_dev(c["X"]), to_dev(c["W"]), to_dev(c["R"])
    y0 = torch.empty((M, N), device=device())
    y1 = torch.full((M, N), float("nan"), device=device())
    st = torch.cuda.current_stream()
    a = (X.data_ptr(), W.data_ptr(), R.data_ptr())
    assert lib.gemm_fwd(*a, y0.data_ptr(), M, K, N, 0, st.cuda_stream) == 0
    say("timing events around 512x768x768")
    for _ in range(3):
        t0, t1 = b.TimingEvent(), b.TimingEvent()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        assert lib.gemm_fwd_ex(*a, y1.data_ptr(), M, K, N, 0, b.opts(-1, None, 0, t0.handle, t1.handle),
                               st.cuda_stream) == 0
        e1.record(st)
        torch.cuda.synchronize()
        kernel_ms, outer_ms = t0.elapsed_ms(t1), e0.elapsed_time(e1)
        say(f"  kernel {kernel_ms * 1e3:.2f} us, torch events around the launch {outer_ms * 1e3:.2f} us")
        assert 0.0 < kernel_ms <= outer_ms * 1.01
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    # recorded as markers around a launch that records no events itself
    m0, m1 = b.TimingEvent(), b.TimingEvent()
    m0.record(st)
    assert lib.gemm_fwd(*a, y1.data_ptr(), M, K, N, 0, st.cuda_stream) == 0
    m1.record(st)
    torch.cuda.synchronize()
    assert m0.elapsed_ms(m1) > 0.0
    assert lib.gemm_timing_event_record(None, st.cuda_stream) == -1
    assert lib.gemm_timing_event_create(None) == -1
    ms = ctypes.c_float()
    assert lib.gemm_timing_elapsed_ms(None, t1.handle, ctypes.byref(ms)) == -1
    assert lib.gemm_timing_elapsed_ms(t0.handle, t1.handle, None) == -1
    assert lib.gemm_timing_event_destroy(None) == 0
