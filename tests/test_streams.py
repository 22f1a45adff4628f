"""Split-K calls on concurrent streams.

The 512 x 3072 x 768 SwiGLU down-projection splits K over two workgroups
per output tile, which meet in the library's static workspace.  Its regions
belong to streams, so calls queued on several streams at once must never
share one: six streams (more than the four regions, so some streams get the
tile without split-K) each queue five calls on their own inputs, and every
result is checked against the oracle.  A shared region would mix two calls'
partial tiles or counters, far outside the tolerance.  A stream without a
region refuses an explicit split-K configuration and runs the library's own
choice on a tile without split-K."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import say, to_dev

pytestmark = pytest.mark.gpu

M, K, N = 512, 3072, 768
STREAMS = 6
CALLS = 5


def test_split_k_calls_on_concurrent_streams():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    cases = [inputs.random_case(700 + i, M, K, N, swiglu=True, residual=True) for i in range(STREAMS)]
    dev_cases = [{k: to_dev(v) for k, v in c.items()} for c in cases]
    outs = [torch.full((M, N), float("nan"), device=dev_cases[0]["G"].device) for _ in range(STREAMS)]
    streams = [torch.cuda.Stream() for _ in range(STREAMS)]
    torch.cuda.synchronize()
    say(f"split-K SwiGLU {M}x{K}x{N} on {STREAMS} streams, {CALLS} calls each")
    for _ in range(CALLS):
        for c, y, st in zip(dev_cases, outs, streams):
            with torch.cuda.stream(st):
                binding.matmul_residual_swiglu_a(c["G"], c["U"], c["W"], c["R"], out=y)
    torch.cuda.synchronize()
    rows = np.arange(0, M, 7, dtype=np.int64)   # every 7th row: all row tiles, a few seconds of oracle
    for i, (c, y) in enumerate(zip(cases, outs)):
        ref, scale = oracle.gemm(c["G"], c["W"], R=c["R"], U=c["U"], rows=rows, want_scale=True)
        res = oracle.compare(y.cpu().numpy()[rows], ref, scale, oracle.TOL_W32)
        say(f"  stream {i}: max err/tol {res['max_ratio']:.3g} fails {res['fails']} of {res['n']}")
        assert res["fails"] == 0, (i, res)


def test_explicit_split_k_config_refused_without_a_region():
    # After split-K calls on four distinct streams every workspace region is
    # owned (by these streams or by earlier ones).  On a fifth stream the
    # library's own choice still runs (on a tile without split-K), while an
    # explicit split-K configuration is refused before anything is enqueued.
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    split_cfg = next(i for i in range(binding.num_configs())
                     if binding.config_name(i) == "32x96x64_w1x2_k2_sp8_pf3_il_ks2_cil_dW")
    c = inputs.random_case(800, M, K, N, swiglu=True, residual=True)
    d = {k: to_dev(v) for k, v in c.items()}
    streams = [torch.cuda.Stream() for _ in range(5)]
    for st in streams[:4]:
        with torch.cuda.stream(st):
            binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"])
    y = torch.full((M, N), float("nan"), device=d["G"].device)
    torch.cuda.synchronize()          # the fill is done before another stream reads y
    with torch.cuda.stream(streams[4]):
        with pytest.raises(binding.GemmError) as err:
            binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], out=y, config=split_cfg)
        assert err.value.status == -7
        assert torch.isnan(y).all()          # nothing was launched
        binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], out=y)
    torch.cuda.synchronize()
    rows = np.arange(3, M, 11, dtype=np.int64)
    ref, scale = oracle.gemm(c["G"], c["W"], R=c["R"], U=c["U"], rows=rows, want_scale=True)
    res = oracle.compare(y.cpu().numpy()[rows], ref, scale, oracle.TOL_W32)
    say(f"  fifth stream, library's choice: max err/tol {res['max_ratio']:.3g} fails {res['fails']}")
    assert res["fails"] == 0, res
