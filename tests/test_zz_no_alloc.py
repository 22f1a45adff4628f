"""gemm_fwd_swiglu_noalloc, the entry point for callers that cannot allocate:
through the C ABI it gives the same bits as gemm_fwd_swiglu_ex with a
caller-provided workspace (same configuration, same arithmetic), and matches
the oracle, on two calls in a row on the library-held array, the second with
a smaller input, both splitting K; and on a shape that does not split K."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import device, say, to_dev

pytestmark = pytest.mark.gpu


def _pair(lib, binding, c, label):
    import torch
    d = {k: to_dev(v) for k, v in c.items()}
    M, K = c["G"].shape
    N = c["W"].shape[1]
    w16 = c["W"].dtype == np.float16
    st = torch.cuda.current_stream().cuda_stream
    args = (d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(), d["R"].data_ptr())
    y_na = torch.full((M, N), float("nan"), device=device())
    y_ws = torch.full((M, N), float("nan"), device=device())
    need = lib.gemm_fwd_workspace_bytes(M, K, N, 1, int(w16), -1)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=device())
    torch.cuda.synchronize()
    say(f"no-alloc {label}: {M}x{K}x{N} w16={w16}, tile {binding.kernel_config(M, K, N, swiglu=True, w16=w16)}, "
        f"workspace {need} bytes")
    assert lib.gemm_fwd_swiglu_noalloc(*args, y_na.data_ptr(), M, K, N, int(w16), st) == 0
    assert lib.gemm_fwd_swiglu_ex(*args, y_ws.data_ptr(), M, K, N, int(w16),
                                  binding.opts(-1, ws.data_ptr() if need else None, need), st) == 0
    torch.cuda.synchronize()
    a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "no-alloc result differs from the workspace call"
    ref, scale = oracle.gemm(c["G"], c["W"], R=c["R"], U=c["U"], want_scale=True)
    res = oracle.compare(a, ref, scale, oracle.TOL_W16 if w16 else oracle.TOL_W32)
    say(f"  max err/tol {res['max_ratio']:.3g} fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res
    return need


def test_no_alloc_matches_workspace_entry_point():
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    # the seq-512 down-projection (K split in two), then a smaller input that
    # also splits K, on the same library-held array
    need1 = _pair(lib, binding, inputs.cfg3(), "first call")
    c2 = inputs.random_case(61, 480, 2048, 800, swiglu=True, residual=True, gate_scale=3.0)
    need2 = _pair(lib, binding, c2, "second, smaller call")
    assert need1 > 0 and need2 > 0
    # a shape the library does not split: the array is not used
    c3 = inputs.random_case(62, 256, 192, 128, swiglu=True, w16=True, residual=True)
    assert _pair(lib, binding, c3, "no split") == 0


def test_no_alloc_argument_errors():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    st = torch.cuda.current_stream().cuda_stream
    x = torch.zeros((8, 8), device=device())
    y = torch.zeros((8, 8), device=device())
    p = x.data_ptr()
    assert lib.gemm_fwd_swiglu_noalloc(p, p, p, p, y.data_ptr(), 8, 8, 8, 2, st) == -4       # weight type
    assert lib.gemm_fwd_swiglu_noalloc(p, p, p, None, y.data_ptr(), 8, 8, 8, 0, st) == -1    # R required
    assert lib.gemm_fwd_swiglu_noalloc(p, p, p, p, y.data_ptr(), 8, 6, 8, 0, st) == -2       # K % 4
    assert lib.gemm_fwd_swiglu_noalloc(p, p, p, p, p, 8, 8, 8, 0, st) == -5                  # Y aliases
