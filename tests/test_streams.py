"""Split-K and its workspace.

The library holds no device memory: configurations that split K over
workgroups exchange their partial tiles through a workspace the caller
passes to the _ex entry points (the binding keeps one zero-filled torch
buffer per stream).  Here:
  * split-K calls queued on six streams at once, each stream with its own
    workspace, all match the oracle;
  * at every shape where the library's choice splits K (the 512 x 3072 x 768
    down-projection with SwiGLU, and with a plain A and f16 W; the lm_head's
    input gradient 512 x 768 x 16384), the choice without a workspace matches
    the oracle on every element and is bitwise reproducible, and so is the
    split-K choice (a plain A with fp32 W is not split either way);
  * an explicit split-K configuration without a workspace is refused before
    anything is enqueued;
  * a completed call leaves the workspace's counters at zero, so one
    zero-fill serves every later call."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import device, say, to_dev

pytestmark = pytest.mark.gpu

M, K, N = 512, 3072, 768
STREAMS = 6
CALLS = 5


def test_split_k_calls_on_concurrent_streams():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert "_ks2" in binding.kernel_config(M, K, N, swiglu=True)
    cases = [inputs.random_case(700 + i, M, K, N, swiglu=True, residual=True) for i in range(STREAMS)]
    dev_cases = [{k: to_dev(v) for k, v in c.items()} for c in cases]
    outs = [torch.full((M, N), float("nan"), device=device()) for _ in range(STREAMS)]
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


@pytest.mark.parametrize("swiglu,w16", [(True, False), (False, False), (True, True), (False, True)])
@pytest.mark.parametrize("use_workspace", [False, True])
def test_long_k_small_grid_with_and_without_workspace(use_workspace, swiglu, w16):
    """512 x 3072 x 768 (the seq-512 down-projection), with SwiGLU and with a
    plain A, fp32 and f16 W: with a workspace the library splits K in two
    (except for a plain A with fp32 W, which 16 x 96 tiles with W in
    registers take over the whole K either way), without one it takes 16 x 96
    tiles over the whole K.  Each: every element against the oracle, and two
    runs bitwise equal."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    c = inputs.cfg3()
    if not swiglu:
        c = {"X": c["G"], "W": c["W"], "R": c["R"]}
    if w16:
        c = dict(c, W=c["W"].astype(np.float16))
    d = {k: to_dev(v) for k, v in c.items()}
    tile = binding.kernel_config(M, K, N, swiglu=swiglu, w16=w16, workspace=use_workspace)
    assert ("_ks" in tile) == (use_workspace and (swiglu or w16)), tile
    say(f"{'SwiGLU' if swiglu else 'plain A'} {M}x{K}x{N} w16={w16} workspace={use_workspace} tile {tile}")
    ys = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), device=device())
        if swiglu:
            binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], out=y, use_workspace=use_workspace)
        else:
            binding.matmul(d["X"], d["W"], d["R"], out=y, use_workspace=use_workspace)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    ref, scale = oracle.gemm(c["G"] if swiglu else c["X"], c["W"], R=c["R"], U=c.get("U"), want_scale=True)
    res = oracle.compare(ys[0], ref, scale, oracle.TOL_W16 if w16 else oracle.TOL_W32)
    say(f"  max err/tol {res['max_ratio']:.3g} fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res


@pytest.mark.parametrize("use_workspace", [False, True])
def test_lm_head_input_gradient_with_and_without_workspace(use_workspace):
    """dX = dY @ W_lm^T (512 x 16384 by 16384 x 768): with a workspace the
    16384-long contraction is split over eight workgroups, without one it is
    not.  Sampled rows (first and last tiles included) against the oracle,
    and two runs bitwise equal."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    Mq, Kq, Nq = 512, 768, 16384
    c = inputs.backward_case(31, Mq, Kq, Nq)
    dY, W = to_dev(c["dY"]), to_dev(c["W"])
    tile = binding.bwd_kernel_config("matmul_t", Mq, Kq, Nq, workspace=use_workspace)
    assert ("_ks8" in tile) == use_workspace, tile
    say(f"lm_head dX workspace={use_workspace} tile {tile}")
    ys = []
    for _ in range(2):
        out = torch.full((Mq, Kq), float("nan"), device=device())
        binding.matmul_t(dY, W, out=out, use_workspace=use_workspace)
        torch.cuda.synchronize()
        ys.append(out.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(0, Mq, 9), np.arange(Mq - 16, Mq)])).astype(np.int64)
    ref, scale = oracle.matmul_t(c["dY"], c["W"], rows=rows, want_scale=True)
    res = oracle.compare(ys[0][rows], ref, scale, oracle.TOL_W32)
    say(f"  max err/tol {res['max_ratio']:.3g} fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res


def test_explicit_split_k_config_needs_a_workspace():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    split_cfg = next(i for i in range(binding.num_configs())
                     if binding.config_name(i) == "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW")
    c = inputs.random_case(800, 64, 512, 96, swiglu=True, residual=True)
    d = {k: to_dev(v) for k, v in c.items()}
    y = torch.full((64, 96), float("nan"), device=device())
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    args = (d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(), d["R"].data_ptr(), y.data_ptr(), 64, 512, 96, 0)
    assert lib.gemm_fwd_swiglu_ex(*args, binding.opts(split_cfg), st) == -8
    torch.cuda.synchronize()
    assert torch.isnan(y).all()          # nothing was launched
    # the same configuration with a workspace runs and matches the oracle
    binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], out=y, config=split_cfg)
    torch.cuda.synchronize()
    ref, scale = oracle.gemm(c["G"], c["W"], R=c["R"], U=c["U"], want_scale=True)
    res = oracle.compare(y.cpu().numpy(), ref, scale, oracle.TOL_W32)
    assert res["fails"] == 0, res


def test_workspace_counters_left_at_zero():
    """After split-K calls complete, the workspace's counter block is zero
    again (its partial slots may hold anything); a fresh zero-filled
    workspace and the reused one give bitwise equal results."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    c = inputs.cfg3()
    d = {k: to_dev(c[k]) for k in ("G", "U", "W", "R")}
    need = lib.gemm_fwd_workspace_bytes(M, K, N, 1, 0, -1)
    assert need == (64 << 10) + 2 * M * N * 4
    ws = torch.zeros(need, dtype=torch.uint8, device=device())
    st = torch.cuda.current_stream().cuda_stream
    ys = []
    for _ in range(3):
        y = torch.empty((M, N), device=device())
        assert lib.gemm_fwd_swiglu_ex(d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(), d["R"].data_ptr(),
                                      y.data_ptr(), M, K, N, 0, binding.opts(-1, ws.data_ptr(), need), st) == 0
        torch.cuda.synchronize()
        assert int(ws[:64 << 10].count_nonzero()) == 0
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint32), ys[2].view(np.uint32))


def test_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in turn: a small
    split-K call (3 output tiles) leaves partial tiles right after the
    counter block, and a later call with 128 tiles must not take them for
    counters.  Every result against the oracle."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    ks2 = next(i for i in range(binding.num_configs())
               if binding.config_name(i) == "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW")
    need = lib.gemm_fwd_workspace_bytes(M, K, N, 1, 0, ks2)
    ws = torch.zeros(need, dtype=torch.uint8, device=device())
    st = torch.cuda.current_stream().cuda_stream
    for seed, (m, k, n) in enumerate([(70, 292, 76), (M, K, N), (33, 260, 52), (M, K, N)]):
        c = inputs.random_case(900 + seed, m, k, n, swiglu=True, residual=True)
        d = {key: to_dev(v) for key, v in c.items()}
        y = torch.full((m, n), float("nan"), device=device())
        say(f"shared workspace call {seed}: {m}x{k}x{n}")
        assert lib.gemm_fwd_swiglu_ex(d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(), d["R"].data_ptr(),
                                      y.data_ptr(), m, k, n, 0, binding.opts(ks2, ws.data_ptr(), need), st) == 0
        torch.cuda.synchronize()
        rows = np.arange(0, m, 5, dtype=np.int64)
        ref, scale = oracle.gemm(c["G"], c["W"], R=c["R"], U=c["U"], rows=rows, want_scale=True)
        res = oracle.compare(y.cpu().numpy()[rows], ref, scale, oracle.TOL_W32)
        assert res["fails"] == 0, (m, k, n, res)
