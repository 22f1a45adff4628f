"""Race check: the shipping library against its verification build.

The kernels order their LDS stages with hand-counted waits (an s_waitcnt
vmcnt(N) that lets the later stages' register loads stay in flight while the
LDS-destination loads of the next stage must have landed), one barrier per
stage ("matmul ve matmul_residual — Tiled Matrix Multiply (Forward)",
"Hızlı Kontrol Listesi": the double-buffered prefetch is race-free by its
barrier), and a split-K exchange ordered by coherent stores and a relaxed
counter.  libgemmfwd_sync.so is the same source built with GEMM_SYNC_CHECK:
every barrier waits for all memory operations first, the LDS-destination
waits wait for everything, and the split-K exchange adds device-scope fences.
The arithmetic and its order are the same, so every output must be equal bit
for bit: in every forward configuration and variant, every backward
configuration and product (and the fused SwiGLU backward), and on the five
workloads in the library's own choice (M = 8192 and 8191 included)."""
import numpy as np
import pytest

from tiled_dense_gemm_matmul_amd import inputs

from _gpu import device, say, to_dev

pytestmark = pytest.mark.gpu


def _libs():
    from tiled_dense_gemm_matmul_amd import binding
    return binding, binding.load_library(), binding.load_sync_check_library()


def _workspace(nbytes):
    import torch
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device())


def _fwd_both(case, cfg=-1):
    """Y from both libraries (same configuration, each with its own zeroed
    workspace)."""
    import torch
    binding, lib, slib = _libs()
    d = {k: to_dev(v) for k, v in case.items()}
    swiglu = "G" in case
    A = case["G"] if swiglu else case["X"]
    M, K = A.shape
    N = case["W"].shape[1]
    w16 = case["W"].dtype == np.float16
    R = d.get("R")
    st = torch.cuda.current_stream().cuda_stream
    need = lib.gemm_fwd_workspace_bytes(M, K, N, int(swiglu), int(w16), cfg)
    assert need >= 0
    outs = []
    for L in (lib, slib):
        ws = _workspace(need)
        y = torch.full((M, N), float("nan"), device=device())
        o = binding.opts(cfg, ws.data_ptr() if need else None, need)
        if swiglu:
            rc = L.gemm_fwd_swiglu_ex(d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(), R.data_ptr(),
                                      y.data_ptr(), M, K, N, int(w16), o, st)
        else:
            rc = L.gemm_fwd_ex(d["X"].data_ptr(), d["W"].data_ptr(), None if R is None else R.data_ptr(),
                               y.data_ptr(), M, K, N, int(w16), o, st)
        assert rc == 0
        outs.append((y, ws))
    torch.cuda.synchronize()
    return outs[0][0], outs[1][0]


def _same(a, b, label):
    import torch
    eq = torch.equal(a.view(torch.int32), b.view(torch.int32))
    if not eq:
        diff = int((a.view(torch.int32) != b.view(torch.int32)).sum())
        say(f"  {label}: {diff} elements differ")
    assert eq, label


@pytest.mark.parametrize("cfg", list(range(40)))
def test_forward_configs(cfg):
    binding, lib, _ = _libs()
    if cfg >= lib.gemm_num_configs():
        pytest.skip("no such configuration")
    name = binding.config_name(cfg)
    for (M, K, N) in [(70, 292, 76), (257, 1024, 196)]:
        for swiglu, w16, resid in [(False, False, True), (False, True, False), (True, False, True),
                                   (True, True, True)]:
            if w16 and not binding.config_takes_w16(cfg):
                continue  # fp32-only tile (W in registers)
            say(f"race check forward {name} {M}x{K}x{N} swiglu={swiglu} w16={w16} resid={resid}")
            c = inputs.random_case(M + K + 3 * swiglu + w16, M, K, N, swiglu=swiglu, w16=w16, residual=resid,
                                   gate_scale=3.0)
            a, b = _fwd_both(c, cfg)
            _same(a, b, f"{name} {M}x{K}x{N} swiglu={swiglu} w16={w16}")


@pytest.mark.parametrize("cfg", list(range(24)))
def test_backward_configs(cfg):
    import torch
    binding, lib, slib = _libs()
    if cfg >= lib.gemm_bwd_num_configs():
        pytest.skip("no such configuration")
    name = binding.bwd_config_name(cfg)
    M, K, N = 292, 68, 292
    st = torch.cuda.current_stream().cuda_stream
    c = inputs.backward_case(77, M, K, N, swiglu=True, acc=True, gate_scale=3.0)
    cx = inputs.backward_case(78, M, K, N, acc=True)
    d = {k: to_dev(v) for k, v in c.items()}
    dx = {k: to_dev(v) for k, v in cx.items()}
    for op in ("t", "t_acc", "at", "at_acc", "at_swiglu", "at_acc_swiglu", "t_swiglu_bwd"):
        say(f"race check backward {name} {op}")
        results = []
        for L in (lib, slib):
            opnum = 1 if op.startswith("t") else 2
            need = L.gemm_bwd_workspace_bytes(opnum, M, K, N, int("swiglu" in op and opnum == 2), cfg)
            assert need >= 0
            ws = _workspace(need)
            o = binding.opts(cfg, ws.data_ptr() if need else None, need)
            acc = 0x2 if "acc" in op else 0
            if op == "t_swiglu_bwd":
                g1 = torch.empty((M, K), device=device())
                g2 = torch.empty((M, K), device=device())
                rc = L.gemm_matmul_t_swiglu_bwd_ex(d["dY"].data_ptr(), d["W"].data_ptr(), d["G"].data_ptr(),
                                                   d["U"].data_ptr(), g1.data_ptr(), g2.data_ptr(), M, K, N, o, st)
                out = torch.cat([g1.reshape(-1), g2.reshape(-1)])
            elif op.startswith("t"):
                out = dx["dX0"].clone()
                rc = L.gemm_matmul_t_ex(dx["dY"].data_ptr(), dx["W"].data_ptr(), out.data_ptr(), M, K, N, acc, o, st)
            elif "swiglu" in op:
                out = d["dW0"].clone()
                rc = L.gemm_matmul_at_swiglu_a_ex(d["G"].data_ptr(), d["U"].data_ptr(), d["dY"].data_ptr(),
                                                  out.data_ptr(), M, K, N, acc, o, st)
            else:
                out = dx["dW0"].clone()
                rc = L.gemm_matmul_at_ex(dx["X"].data_ptr(), dx["dY"].data_ptr(), out.data_ptr(), M, K, N, acc, o, st)
            assert rc == 0
            results.append((out, ws))
        torch.cuda.synchronize()
        _same(results[0][0], results[1][0], f"{name} {op}")


def test_workloads_library_choice():
    """The five workloads, in the configuration the library picks with a
    workspace (the one bench.py times)."""
    c1, c2, c3, c4, c5 = inputs.cfg1(), inputs.cfg2(), inputs.cfg3(), inputs.cfg4(), inputs.cfg5()
    cases = [("cfg1", c1), ("cfg2 +R", c2), ("cfg2", {"X": c2["X"], "W": c2["W"]}), ("cfg3", c3),
             ("cfg4 lm_head", {"X": c4["X"], "W": c4["W_lm"]}), ("cfg4b gate/up", {"X": c4["X"], "W": c4["W_gu"]})]
    for M in (8192, 8191):
        cases.append((f"cfg5a M={M}", {"G": np.ascontiguousarray(c5["G"][:M]), "U": np.ascontiguousarray(c5["U"][:M]),
                                       "W": c5["W_down"], "R": np.ascontiguousarray(c5["R"][:M])}))
        cases.append((f"cfg5b M={M}", {"X": np.ascontiguousarray(c5["X"][:M]), "W": c5["W_lm"]}))
    for label, c in cases:
        say(f"race check workload {label}")
        a, b = _fwd_both(c)
        _same(a, b, label)
        del a, b
