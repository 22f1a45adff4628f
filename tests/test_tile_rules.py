"""Parity in the configurations that the tile-choice rules for mid-size and
batch-size grids pick (each test first checks that the rule picked it):
the forward 128 x 64, 128 x 48 and 64 x 64 tiles, the forward 16 x 48 and
16 x 96 tiles with W in registers (small grids, fp32 W; SwiGLU too), and the
backward 128 x 64 (transposed B), 48 x 48 (one-round dW over a long
contraction) and 32 x 96 with dY in registers (dW, SwiGLU too) tiles.  Large outputs are compared on sampled rows that include
the last tile's rows."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import check, run, say, to_dev

pytestmark = pytest.mark.gpu


def _rows(M, seed, count=48, tail=128):
    rng = np.random.default_rng(seed)
    start = max(M - tail, 0)
    return np.unique(np.concatenate([rng.choice(max(start, 1), size=min(count, max(start, 1)), replace=False),
                                     np.arange(start, M)])).astype(np.int64)


@pytest.mark.parametrize("M,K,N,w16,resid,tile", [
    (512, 768, 8192, True, False, "128x64x32_w2x2_sp4_pf3_il_dA"),
    (8192, 768, 768, False, True, "128x64x32_w2x2_sp4_pf3_il_dA"),
    (512, 768, 2048, True, False, "64x64x64_w2x2_sp4_dAW"),
    (512, 768, 3072, True, False, "128x48x32_w2x1_k2_sp4_pf3_il_dA"),
    (2048, 768, 772, True, True, "128x48x32_w2x1_k2_sp4_pf3_il_dA"),
    # small grids with fp32 W: W in the compute waves' registers
    (512, 1024, 1024, False, False, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (250, 768, 768, False, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (256, 768, 772, False, True, "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"),
    (2048, 768, 772, False, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (2048, 768, 768, False, False, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (2040, 768, 760, False, True, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (512, 2000, 768, False, False, "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"),
    # few rows against a wide W: no 128-row tiles at 64 rows or fewer, no
    # 64-row tiles at 32 or fewer (48 with fp32 W beyond one round)
    (16, 768, 50304, True, False, "16x48x128_k4_sp4_dAW"),
    (1, 768, 50304, False, False, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (48, 768, 50304, False, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (17, 768, 16388, False, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (64, 768, 50304, True, False, "64x64x64_w2x2_sp4_dAW"),
    # a 128 x 128 grid that fills under 70% of its rounds (576 tiles)
    (3072, 768, 3072, True, False, "128x64x32_w2x2_sp4_pf3_il_dA"),
    (3070, 772, 3068, True, True, "128x64x32_w2x2_sp4_pf3_il_dA"),
    # a 128 x 64 grid that fills under 70% of its rounds (576 tiles): 32 x 192
    # with fp32 W, 128 x 48 with f16 W, else 64 x 64 below 60% (648 tiles
    # keep 128 x 64)
    (3072, 768, 1536, False, False, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (3072, 768, 1536, True, False, "128x48x32_w2x1_k2_sp4_pf3_il_dA"),
    (3001, 768, 1540, True, True, "64x64x64_w2x2_sp4_dAW"),
    (2304, 768, 2304, True, False, "128x64x32_w2x2_sp4_pf3_il_dA"),
    # a 64 x 64 grid that fills under 70% of its rounds (576 tiles): 64 x 48
    # where that grid fills whole rounds of three per CU, else 32 x 192 with
    # fp32 W or 128 x 48 with f16 W where that grid fills its rounds
    (1536, 768, 1536, False, False, "64x48x64_w2x1_k2_sp4_pf3_il_dA"),
    (1530, 768, 1532, True, True, "64x48x64_w2x1_k2_sp4_pf3_il_dA"),
    (2304, 768, 1152, True, False, "128x48x32_w2x1_k2_sp4_pf3_il_dA"),
    (2304, 768, 1152, False, False, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (448, 768, 6528, True, False, "64x64x64_w2x2_sp4_dAW"),
    # one whole round of 64 x 64 tiles over a long contraction: K split in two
    (1024, 4096, 1024, False, False, "64x64x64_w2x2_sp4_ks2_dAW"),
    (1000, 4100, 1020, True, True, "64x64x64_w2x2_sp4_ks2_dAW"),
    # few columns: no tile more than twice as wide as the columns it covers
    (8192, 768, 48, False, False, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (32768, 768, 64, False, True, "64x64x64_w2x2_sp4_dAW"),
    (8191, 772, 64, True, True, "64x48x64_w2x1_k2_sp4_pf3_il_dA"),
])
def test_forward_rule(M, K, N, w16, resid, tile):
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.kernel_config(M, K, N, w16=w16) == tile
    say(f"forward {M}x{K}x{N} w16={w16} R={resid} -> {tile}")
    c = inputs.random_case(1000 + M + N, M, K, N, w16=w16, residual=resid)
    y = run(c).cpu().numpy()
    rows = _rows(M, 7)
    check(c, y[rows], rows=rows, label=f"{M}x{K}x{N} {tile}")


@pytest.mark.parametrize("M,K,N,ws,tile", [
    (512, 1536, 768, True, "16x96x128_w1x2_k2_sp8_pf2_il_wr4"),
    (480, 2048, 800, True, "16x192x128_w1x4_sp4_pf3_il_ks2_wr4"),
    (200, 2500, 772, False, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (768, 768, 2048, True, "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"),
    (1000, 768, 1532, True, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (8192, 1024, 768, True, "32x384x64_w1x4_sp4_pf3_il_dA_wr2"),
    (8191, 1024, 772, True, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (384, 2048, 768, False, "16x96x128_w1x2_k2_sp8_pf2_il_wr4"),
    (8192, 3072, 32, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
    (3072, 768, 1536, True, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (2300, 772, 1148, True, "32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    (8190, 3076, 36, True, "16x48x128_k4_sp4_pf3_il_dA_wr2"),
])
def test_forward_rule_swiglu_fp32(M, K, N, ws, tile):
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.kernel_config(M, K, N, swiglu=True, workspace=ws) == tile
    say(f"forward SwiGLU {M}x{K}x{N} workspace={ws} -> {tile}")
    c = inputs.random_case(2000 + M + N, M, K, N, swiglu=True, residual=True, gate_scale=3.0)
    y = binding.matmul_residual_swiglu_a(to_dev(c["G"]), to_dev(c["U"]), to_dev(c["W"]), to_dev(c["R"]),
                                         use_workspace=ws)
    torch.cuda.synchronize()
    check(c, y.cpu().numpy(), label=f"{M}x{K}x{N} {tile}")


@pytest.mark.parametrize("M,K,N,swiglu,w16,tile", [
    (77, 4100, 500, False, False, "16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"),
    (63, 3076, 2044, False, False, "16x48x128_k4_sp4_pf3_il_ks2_dA_wr2"),
    (29, 3072, 2044, True, False, "16x96x128_w1x2_k2_sp4_pf3_il_ks4_dA_wr4"),
    (175, 3076, 1020, True, False, "16x96x128_w1x2_k2_sp4_pf3_il_ks2_dA_wr4"),
    (61, 3076, 2044, True, False, "16x192x128_w1x4_sp4_pf3_il_ks4_wr4"),
    # binary16 W: LDS-staged tiles
    (77, 3076, 2044, False, True, "16x48x128_k4_sp4_ks2_dAW"),
    (17, 3076, 500, True, True, "16x48x128_k4_sp4_ks4_dAW"),
    (255, 3076, 2044, True, True, "32x48x128_k4_sp8_pf2_ks2_dAW"),
    (17, 3076, 2044, False, True, "32x48x128_k4_sp8_pf2_ks4_dAW"),
    (45, 3076, 2044, True, True, "32x96x128_w1x2_k2_sp8_pf3_il_ks4_cil_dAW"),
])
def test_forward_split_small_outputs(M, K, N, swiglu, w16, tile):
    # small outputs over a long contraction: the 16- or 32-row tiles with K
    # split over two or four workgroups when there is a workspace (the whole
    # K without one); both choices on every element against the oracle, the
    # split one run twice and bitwise equal
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.kernel_config(M, K, N, swiglu=swiglu, w16=w16) == tile
    assert "_ks" not in binding.kernel_config(M, K, N, swiglu=swiglu, w16=w16, workspace=False)
    c = inputs.random_case(3000 + M + N, M, K, N, swiglu=swiglu, w16=w16, residual=swiglu, gate_scale=3.0)
    d = {k: to_dev(v) for k, v in c.items()}
    ys = []
    for ws in (True, True, False):
        if swiglu:
            y = binding.matmul_residual_swiglu_a(d["G"], d["U"], d["W"], d["R"], use_workspace=ws)
        else:
            y = binding.matmul(d["X"], d["W"], use_workspace=ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    say(f"forward {'SwiGLU ' if swiglu else ''}{M}x{K}x{N} -> {tile}")
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    check(c, ys[0], label=f"{M}x{K}x{N} {tile}")
    check(c, ys[2], label=f"{M}x{K}x{N} without a workspace")


def _cmp(y, ref, scale, label):
    res = oracle.compare(y, ref, scale, oracle.TOL_W32)
    say(f"  {label}: max err/tol {res['max_ratio']:.4g}, fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res


@pytest.mark.parametrize("M,K,N,tile", [
    (175, 1020, 8196, "16x48x128_k4_sp4_ks2_dAW"),
    (17, 500, 2052, "16x48x128_k4_sp4_ks4_dAW"),
    (17, 500, 4100, "16x48x128_k4_sp4_ks8_dAW"),
    (131, 1020, 8196, "32x48x128_k4_sp8_pf2_ks2_dAW"),
    (45, 1020, 2052, "32x48x128_k4_sp8_pf2_ks4_dAW"),
    (17, 772, 4100, "32x48x128_k4_sp8_pf2_ks8_dAW"),
])
def test_backward_matmul_t_split_small_outputs(M, K, N, tile):
    # dX = dY @ W^T over a long contraction onto a small grid: K split over
    # two, four or eight workgroups with a workspace (not without one); both
    # against the oracle, the split one twice and bitwise equal; then the
    # same split with the SwiGLU backward in its epilogue (after the
    # reduction) against the composition of the two oracles
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    from test_backward import check_fused, fused_ref
    assert binding.bwd_kernel_config("matmul_t", M, K, N) == tile
    assert "_ks" not in binding.bwd_kernel_config("matmul_t", M, K, N, workspace=False)
    c = inputs.backward_case(40 + M + N, M, K, N, swiglu=True, gate_scale=3.0)
    dY, W = to_dev(c["dY"]), to_dev(c["W"])
    ys = []
    for ws in (True, True, False):
        y = binding.matmul_t(dY, W, use_workspace=ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    ref, scale = oracle.matmul_t(c["dY"], c["W"], want_scale=True)
    _cmp(ys[0], ref, scale, f"matmul_t {M}x{K}x{N} {tile}")
    _cmp(ys[2], ref, scale, f"matmul_t {M}x{K}x{N} without a workspace")
    dg, du = binding.matmul_t_swiglu_backward(dY, W, to_dev(c["G"]), to_dev(c["U"]))
    torch.cuda.synchronize()
    rg, ru, bg, bu = fused_ref(c, c["G"], c["U"])
    check_fused(dg.cpu().numpy(), rg, bg, "dGATE")
    check_fused(du.cpu().numpy(), ru, bu, "dUP")


@pytest.mark.parametrize("M,K,N,tile", [(32768, 64, 768, "64x64x64_w2x2_sp4"),
                                        (32767, 20, 772, "64x48x64_w2x1_k2_sp4_pf3_il_dA"),
                                        (16383, 96, 3076, "64x48x64_w2x1_k2_sp4_pf3_il_dA")])
def test_backward_matmul_t_narrow_output(M, K, N, tile):
    # dX = dY @ W^T onto a narrow dX (a layer with few inputs) over many
    # tokens: no tile more than twice as wide as the columns it covers
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.bwd_kernel_config("matmul_t", M, K, N) == tile
    c = inputs.backward_case(21 + K, M, K, N)
    dX = binding.matmul_t(to_dev(c["dY"]), to_dev(c["W"]))
    torch.cuda.synchronize()
    rows = _rows(M, 12)
    ref, scale = oracle.matmul_t(c["dY"], c["W"], rows=rows, want_scale=True)
    _cmp(dX.cpu().numpy()[rows], ref, scale, f"matmul_t {M}x{K}x{N} {tile}")


@pytest.mark.parametrize("M,K,N", [(3072, 3072, 768), (3001, 3052, 772)])
def test_backward_matmul_t_partial_round(M, K, N):
    # dX = dY @ W^T onto 3072 x 3072 (and a ragged neighbour), where 128 x 128
    # tiles would fill under 70% of their rounds: 128 x 64
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.bwd_kernel_config("matmul_t", M, K, N) == "128x64x32_w2x2_sp4_pf3_il_dA"
    c = inputs.backward_case(41 + K, M, K, N)
    dX = binding.matmul_t(to_dev(c["dY"]), to_dev(c["W"]))
    torch.cuda.synchronize()
    rows = _rows(M, 17)
    ref, scale = oracle.matmul_t(c["dY"], c["W"], rows=rows, want_scale=True)
    _cmp(dX.cpu().numpy()[rows], ref, scale, f"matmul_t {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(512, 4352, 1536), (1023, 4348, 1540)])
def test_backward_matmul_t_partial_round_64x48(M, K, N):
    # dX = dY @ W^T where the 64 x 64 (128 x 64) grid would fill under 60%
    # of its rounds: 64 x 48
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.bwd_kernel_config("matmul_t", M, K, N) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    c = inputs.backward_case(43 + K, M, K, N)
    dX = binding.matmul_t(to_dev(c["dY"]), to_dev(c["W"]))
    torch.cuda.synchronize()
    rows = _rows(M, 19)
    ref, scale = oracle.matmul_t(c["dY"], c["W"], rows=rows, want_scale=True)
    _cmp(dX.cpu().numpy()[rows], ref, scale, f"matmul_t {M}x{K}x{N}")


def test_backward_matmul_t_128x64():
    # dX = dY @ W^T for 8192 tokens, 768 outputs, 768 inputs
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    M, K, N = 8192, 768, 768
    assert binding.bwd_kernel_config("matmul_t", M, K, N) == "128x64x32_w2x2_sp4_pf3_il_dA"
    c = inputs.backward_case(11, M, K, N)
    dX = binding.matmul_t(to_dev(c["dY"]), to_dev(c["W"]))
    torch.cuda.synchronize()
    rows = _rows(M, 8)
    ref, scale = oracle.matmul_t(c["dY"], c["W"], rows=rows, want_scale=True)
    _cmp(dX.cpu().numpy()[rows], ref, scale, "matmul_t 8192x768x768")


@pytest.mark.parametrize("M,K,N,ks", [(8192, 768, 768, 2), (2051, 760, 764, 2), (4099, 508, 516, 4)])
def test_backward_matmul_at_48x48_long_contraction(M, K, N, ks):
    # dW = X^T @ dY over 2048 tokens or more onto a small grid of 48 x 48
    # tiles: K split over ks workgroups with a workspace (ragged splits where
    # the token count is), the whole K per workgroup without one; both
    # against the oracle, and accumulating into dW0 with the split
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    c = inputs.backward_case(12 + N, M, K, N)
    X, dY = to_dev(c["X"]), to_dev(c["dY"])
    rows = _rows(K, 9, count=32, tail=48)
    ref, scale = oracle.matmul_at(c["X"], c["dY"], rows=rows, want_scale=True)
    for ws, tile in ((True, f"48x48x64_k4_sp4_pf2_ks{ks}_dAW"), (False, "48x48x64_k4_sp4_pf3_dAW")):
        assert binding.bwd_kernel_config("matmul_at", M, K, N, workspace=ws) == tile
        dW = binding.matmul_at(X, dY, use_workspace=ws)
        torch.cuda.synchronize()
        _cmp(dW.cpu().numpy()[rows], ref, scale, f"matmul_at {M}x{K}x{N} {tile}")
    dW0 = inputs.backward_case(13 + N, M, K, N, acc=True)["dW0"]
    out = to_dev(dW0)
    binding.matmul_at(X, dY, out=out, acc=True)
    torch.cuda.synchronize()
    ref, scale = oracle.matmul_at(c["X"], c["dY"], Y0=dW0, rows=rows, want_scale=True)
    _cmp(out.cpu().numpy()[rows], ref, scale, f"matmul_at_acc {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(1024, 3072, 3072), (1023, 3076, 3068), (1024, 2304, 3072), (1000, 2300, 3068)])
def test_backward_matmul_at_w_in_registers_partial_round(M, K, N):
    # dW over 1024 tokens onto 3072 x 3072 (and 2304 x 3072), where 128 x 128
    # (128 x 192) tiles would fill under 70% of their rounds: dY in registers
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    assert binding.bwd_kernel_config("matmul_at", M, K, N) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    c = inputs.backward_case(31 + N, M, K, N)
    dW = binding.matmul_at(to_dev(c["X"]), to_dev(c["dY"]))
    torch.cuda.synchronize()
    rows = _rows(K, 13, count=64, tail=96)
    ref, scale = oracle.matmul_at(c["X"], c["dY"], rows=rows, want_scale=True)
    _cmp(dW.cpu().numpy()[rows], ref, scale, f"matmul_at {M}x{K}x{N}")


@pytest.mark.parametrize("tokens", [512, 8192])
@pytest.mark.parametrize("swiglu", [False, True])
def test_backward_matmul_at_w_in_registers(swiglu, tokens):
    # dW over 512 and 8192 tokens: gate/up's 768 x 3072 and the SwiGLU
    # down-projection's 3072 x 768 (dY loaded into registers)
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    M, K, N = (tokens, 3072, 768) if swiglu else (tokens, 768, 3072)
    assert binding.bwd_kernel_config("matmul_at", M, K, N, swiglu=swiglu) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    c = inputs.backward_case(14 + swiglu, M, K, N, swiglu=swiglu, gate_scale=3.0)
    if swiglu:
        dW = binding.matmul_at_swiglu_a(to_dev(c["G"]), to_dev(c["U"]), to_dev(c["dY"]))
    else:
        dW = binding.matmul_at(to_dev(c["X"]), to_dev(c["dY"]))
    torch.cuda.synchronize()
    rows = _rows(K, 11, count=64, tail=96)
    ref, scale = oracle.matmul_at(c["G"] if swiglu else c["X"], c["dY"], U=c.get("U"), rows=rows, want_scale=True)
    _cmp(dW.cpu().numpy()[rows], ref, scale, f"matmul_at{'_swiglu_a' if swiglu else ''} {M}x{K}x{N}")
