"""The backward linear family on the GPU against the oracle: matmul_t and
matmul_t_acc (dX = dY W^T), matmul_at and matmul_at_acc (dW = X^T dY),
matmul_at_swiglu_a and matmul_at_acc_swiglu_a (dW = (silu(G) U)^T dY), on
ragged shapes that leave partial tiles in every dimension, in every
configuration of the backward table, at the seq-512 model's shapes (output
rows sampled where the oracle would be slow), and on the degenerate shapes."""
import numpy as np
import pytest

import oracle
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import device, say, to_dev

pytestmark = pytest.mark.gpu

OPS = ["t", "t_acc", "at", "at_acc", "at_swiglu", "at_acc_swiglu"]


def gpu(case, op, config=None):
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    acc = "acc" in op
    if op.startswith("t"):
        out = to_dev(case["dX0"]) if acc else None
        y = binding.matmul_t(to_dev(case["dY"]), to_dev(case["W"]), out=out, acc=acc, config=config)
    elif "swiglu" in op:
        out = to_dev(case["dW0"]) if acc else None
        y = binding.matmul_at_swiglu_a(to_dev(case["G"]), to_dev(case["U"]), to_dev(case["dY"]), out=out, acc=acc,
                                       config=config)
    else:
        out = to_dev(case["dW0"]) if acc else None
        y = binding.matmul_at(to_dev(case["X"]), to_dev(case["dY"]), out=out, acc=acc, config=config)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def ref(case, op, rows=None):
    acc = "acc" in op
    if op.startswith("t"):
        return oracle.matmul_t(case["dY"], case["W"], Y0=case["dX0"] if acc else None, rows=rows, want_scale=True)
    A = case["G"] if "swiglu" in op else case["X"]
    return oracle.matmul_at(A, case["dY"], Y0=case["dW0"] if acc else None, U=case.get("U"), rows=rows,
                            want_scale=True)


def check(case, op, y, rows=None, label=""):
    y_ref, b = ref(case, op, rows=rows)
    if rows is not None:
        y = y[rows]
    res = oracle.compare(y, y_ref, b, oracle.TOL_W32)
    say(f"  {label} {op}: max err/tol = {res['max_ratio']:.4g}, fails = {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res


def case_for(seed, M, K, N, op):
    return inputs.backward_case(seed, M, K, N, swiglu="swiglu" in op, acc="acc" in op, gate_scale=3.0)


@pytest.mark.parametrize("op", OPS)
def test_ragged(op):
    for (M, K, N) in [(77, 132, 100), (130, 68, 196), (33, 260, 52), (300, 96, 36), (5, 4, 4)]:
        say(f"backward {op} M={M} K={K} N={N}")
        case = case_for(M * 13 + K, M, K, N, op)
        check(case, op, gpu(case, op), label=f"{M}x{K}x{N}")


@pytest.mark.parametrize("op", OPS)
def test_every_backward_config(op):
    from tiled_dense_gemm_matmul_amd import binding
    for (M, K, N) in [(77, 132, 100), (130, 68, 196)]:
        case = case_for(M * 17 + N, M, K, N, op)
        for cfg in range(binding.bwd_num_configs()):
            name = binding.bwd_config_name(cfg)
            say(f"backward {op} config {name} M={M} K={K} N={N}")
            check(case, op, gpu(case, op, config=cfg), label=name)


# seq-512 model shapes (forward names M x K x N): the backward of qkvo, of the
# FFN down-projection (dH from W_down, dW_down from the recomputed SwiGLU
# activation), of gate/up, and of the lm_head (its dX and dW).
MODEL = [
    ("t", 512, 768, 768), ("t", 512, 3072, 768), ("t", 512, 768, 3072), ("t_acc", 512, 768, 16384),
    ("at", 512, 768, 768), ("at_acc", 512, 768, 3072), ("at_swiglu", 512, 3072, 768), ("at", 512, 768, 16384),
]


@pytest.mark.parametrize("op,M,K,N", MODEL)
def test_model_shapes(op, M, K, N):
    say(f"backward model shape {op} M={M} K={K} N={N}")
    case = case_for(M + K + N, M, K, N, op)
    y = gpu(case, op)
    out_rows = M if op.startswith("t") else K
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, out_rows - 1], rng.choice(out_rows, 24, replace=False)]))
    check(case, op, y, rows=rows, label=f"{M}x{K}x{N}")


def test_degenerate():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    dev = device()
    # empty contraction: zeros, or the output unchanged when accumulating
    dY = torch.empty((6, 0), device=dev)
    W = torch.empty((8, 0), device=dev)
    y = binding.matmul_t(dY, W)
    torch.cuda.synchronize()
    assert y.shape == (6, 8) and torch.count_nonzero(y).item() == 0
    prev = torch.randn((6, 8), device=dev)
    keep = prev.clone()
    binding.matmul_t(dY, W, out=prev, acc=True)
    torch.cuda.synchronize()
    assert torch.equal(prev, keep)
    X = torch.empty((0, 8), device=dev)
    dY0 = torch.empty((0, 12), device=dev)
    y = binding.matmul_at(X, dY0)
    torch.cuda.synchronize()
    assert y.shape == (8, 12) and torch.count_nonzero(y).item() == 0
    # empty outputs: nothing to do
    assert binding.matmul_t(torch.empty((0, 4), device=dev), torch.randn((8, 4), device=dev)).shape == (0, 8)
    assert binding.matmul_at(torch.randn((5, 0), device=dev), torch.randn((5, 4), device=dev)).shape == (0, 4)


def test_adjoint_on_gpu():
    """<X W, dY> = <X, dY W^T> = <W, X^T dY> with all three products from the
    library, in float64 on the host."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    rng = np.random.default_rng(21)
    M, K, N = 256, 384, 320
    X = rng.standard_normal((M, K), dtype=np.float32)
    W = rng.standard_normal((K, N), dtype=np.float32) * np.float32(0.05)
    dY = rng.standard_normal((M, N), dtype=np.float32)
    fwd = binding.matmul(to_dev(X), to_dev(W)).cpu().numpy().astype(np.float64)
    dX = binding.matmul_t(to_dev(dY), to_dev(W)).cpu().numpy().astype(np.float64)
    dW = binding.matmul_at(to_dev(X), to_dev(dY)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    lhs = float(np.sum(fwd * dY))
    mag = float(np.sum(np.abs(X.astype(float)) @ np.abs(W.astype(float)) * np.abs(dY)))
    assert abs(float(np.sum(dX * X)) - lhs) <= 1e-5 * mag
    assert abs(float(np.sum(dW * W)) - lhs) <= 1e-5 * mag


def test_misaligned_and_flags_are_rejected():
    import ctypes
    from tiled_dense_gemm_matmul_amd import binding
    lib = binding.load_library()
    dev = device()
    import torch
    dY = torch.randn((8, 8), device=dev)
    W = torch.randn((8, 8), device=dev)
    out = torch.empty((8, 8), device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    # W_F16 is not a backward flag
    assert lib.gemm_matmul_t(dY.data_ptr(), W.data_ptr(), out.data_ptr(), 8, 8, 8, 0x1, st) == -4
    # output aliasing an input
    assert lib.gemm_matmul_at(dY.data_ptr(), W.data_ptr(), dY.data_ptr(), 8, 8, 8, 0, st) == -5
    # K % 4
    assert lib.gemm_matmul_t(dY.data_ptr(), W.data_ptr(), out.data_ptr(), 8, 6, 8, 0, st) == -2
    # misaligned pointer
    assert lib.gemm_matmul_at(ctypes.c_void_p(dY.data_ptr() + 4), W.data_ptr(), out.data_ptr(), 8, 8, 8, 0, st) == -3


# --- the fused SwiGLU backward: matmul_t's dH turned into dGATE, dUP in the epilogue ---

def fused_ref(case, G, U, rows=None):
    """The composition of the two pinned oracles, with the bound it implies:
    dH within the GEMM tolerance, propagated through the element-wise
    derivatives, plus the element-wise kernels' own tolerance."""
    from oracle import activation as OA
    dh, b = oracle.matmul_t(case["dY"], case["W"], rows=rows, want_scale=True)
    g = G if rows is None else G[rows]
    u = U if rows is None else U[rows]
    dg, du, mg, mu = OA.ffn_swiglu_backward(dh, g, u)
    x = g.astype(np.float64)
    s = OA.sigmoid(x)
    dh_err = oracle.TOL_W32[0] * b + oracle.TOL_W32[1]
    bg = np.abs(u) * s * (1.0 + np.abs(x) * (1.0 - s)) * dh_err + OA.TOL[0] * mg
    bu = np.abs(x) * s * dh_err + OA.TOL[0] * mu
    return dg, du, bg, bu


def check_fused(y, ref, bound, label):
    err = np.abs(np.asarray(y, np.float64) - ref)
    ratio = np.where(bound > 0, err / np.maximum(bound, 1e-300), np.where(err == 0, 0.0, np.inf))
    fails = int(np.count_nonzero(~(ratio <= 1.0)))
    say(f"  {label}: max err/tol {float(np.max(ratio)) if ratio.size else 0.0:.3g}, fails {fails} of {ratio.size}")
    assert fails == 0


def fused_case(seed, M, K, N):
    c = inputs.backward_case(seed, M, K, N)
    rng = np.random.default_rng(seed + 1)
    G = (rng.standard_normal((M, K), dtype=np.float32) * np.float32(3.0))
    U = rng.standard_normal((M, K), dtype=np.float32)
    return c, G, U


@pytest.mark.parametrize("M,K,N", [(77, 132, 100), (130, 68, 196), (33, 260, 52), (512, 3072, 768)])
def test_fused_swiglu_backward(M, K, N):
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    say(f"fused swiglu backward M={M} K={K} N={N}")
    c, G, U = fused_case(M * 3 + K, M, K, N)
    dg, du = binding.matmul_t_swiglu_backward(to_dev(c["dY"]), to_dev(c["W"]), to_dev(G), to_dev(U))
    torch.cuda.synchronize()
    rows = None if M * K < 1e6 else np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 30)]))
    rg, ru, bg, bu = fused_ref(c, G, U, rows=rows)
    sel = slice(None) if rows is None else rows
    check_fused(dg.cpu().numpy()[sel], rg, bg, "dGATE")
    check_fused(du.cpu().numpy()[sel], ru, bu, "dUP")


def test_fused_swiglu_backward_every_config_and_in_place():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    M, K, N = 130, 68, 196
    c, G, U = fused_case(5, M, K, N)
    rg, ru, bg, bu = fused_ref(c, G, U)
    for cfg in range(binding.bwd_num_configs()):
        say(f"fused swiglu backward config {binding.bwd_config_name(cfg)}")
        dg, du = binding.matmul_t_swiglu_backward(to_dev(c["dY"]), to_dev(c["W"]), to_dev(G), to_dev(U), config=cfg)
        torch.cuda.synchronize()
        check_fused(dg.cpu().numpy(), rg, bg, f"dGATE {binding.bwd_config_name(cfg)}")
        check_fused(du.cpu().numpy(), ru, bu, f"dUP {binding.bwd_config_name(cfg)}")
    # the gradients written over GATE and UP themselves
    g, u = to_dev(G), to_dev(U)
    binding.matmul_t_swiglu_backward(to_dev(c["dY"]), to_dev(c["W"]), g, u, grad_gate=g, grad_up=u)
    torch.cuda.synchronize()
    check_fused(g.cpu().numpy(), rg, bg, "dGATE over GATE")
    check_fused(u.cpu().numpy(), ru, bu, "dUP over UP")
    # empty contraction: dH = 0, both gradients zero
    dev = device()
    z = torch.empty((6, 0), device=dev)
    dg, du = binding.matmul_t_swiglu_backward(z, torch.empty((8, 0), device=dev), torch.randn((6, 8), device=dev),
                                              torch.randn((6, 8), device=dev))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dg).item() == 0 and torch.count_nonzero(du).item() == 0
