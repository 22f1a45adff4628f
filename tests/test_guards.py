"""No kernel reads outside its inputs or writes outside its outputs.

The page's kernels rely on WebGPU robust access for out-of-range reads
("matmul ve matmul_residual — Tiled Matrix Multiply (Forward)", "Code
Review / Bulgu 1"); this library instead stages masked elements from
offsets past its buffer descriptors' ends (and, for LDS-destination loads,
from rebased per-stage descriptors), so the masking is shown here for every
kernel instantiation: every read-only input gets NaN neighbours (a single
stray read turns a result NaN or, through nan_guard, zero, and fails
parity), every output and every array updated in place gets sentinel bands
that must survive, and every result is checked against the oracle.  Shapes
leave partial tiles in every dimension, and the contractions are at least
two 128-deep stages long plus a ragged part, so that both the whole-stage
and the partial-stage load paths run."""
import numpy as np
import pytest

import oracle
from oracle import activation as OA
from oracle import loss as OL
from tiled_dense_gemm_matmul_amd import inputs

from _gpu import check, device, say
from test_backward import check as check_bwd
from test_backward import check_fused, fused_case, fused_ref

pytestmark = pytest.mark.gpu

PAD = 4096
SENTINEL = -777.0


def poisoned(a):
    """Device copy of the read-only array a with NaN neighbours."""
    import torch
    flat = np.ascontiguousarray(a).reshape(-1)
    dt = {np.dtype(np.float32): torch.float32, np.dtype(np.float16): torch.float16}[flat.dtype]
    buf = torch.full((2 * PAD + flat.size,), float("nan"), dtype=dt, device=device())
    buf[PAD:PAD + flat.size] = torch.from_numpy(flat).to(device())
    return buf[PAD:PAD + flat.size].view(*a.shape)


class Banded:
    """An fp32 device array inside sentinel bands (initial contents `init`,
    or the sentinel)."""

    def __init__(self, shape, init=None, sentinel=SENTINEL):
        import torch
        self.n = int(np.prod(shape))
        self.sentinel = sentinel
        self.buf = torch.full((2 * PAD + self.n,), sentinel, dtype=torch.float32, device=device())
        if init is not None:
            self.buf[PAD:PAD + self.n] = torch.from_numpy(np.ascontiguousarray(init, np.float32).reshape(-1)).to(
                device())
        self.view = self.buf[PAD:PAD + self.n].view(*shape)

    def result(self, label):
        import torch
        torch.cuda.synchronize()
        host = self.buf.cpu().numpy()
        assert np.all(host[:PAD] == self.sentinel) and np.all(host[PAD + self.n:] == self.sentinel), \
            f"{label}: write outside the output"
        return host[PAD:PAD + self.n].reshape(self.view.shape)


def _fwd_configs():
    from tiled_dense_gemm_matmul_amd import binding
    return binding.num_configs()


@pytest.mark.parametrize("cfg", [None] + list(range(40)))
def test_forward_every_config(cfg):
    from tiled_dense_gemm_matmul_amd import binding
    if cfg is not None and cfg >= binding.num_configs():
        pytest.skip("no such configuration")
    M, K, N = 70, 292, 76
    name = "library's choice" if cfg is None else binding.config_name(cfg)
    for swiglu, w16, resid in [(False, False, False), (False, False, True), (False, True, False),
                               (False, True, True), (True, False, True), (True, True, True)]:
        if w16 and cfg is not None and not binding.config_takes_w16(cfg):
            continue  # fp32-only tile (W in registers)
        say(f"guards forward {name} M={M} K={K} N={N} swiglu={swiglu} w16={w16} resid={resid}")
        c = inputs.random_case(7 + 2 * swiglu + w16, M, K, N, swiglu=swiglu, w16=w16, residual=resid,
                               gate_scale=2.0)
        W = poisoned(c["W"])
        R = poisoned(c["R"]) if resid else None
        y = Banded((M, N))
        if swiglu:
            binding.matmul_residual_swiglu_a(poisoned(c["G"]), poisoned(c["U"]), W, R, out=y.view, config=cfg)
        else:
            binding.matmul(poisoned(c["X"]), W, R, out=y.view, config=cfg)
        yy = y.result(name)
        assert np.all(np.isfinite(yy)), f"{name}: NaN from outside an input reached Y"
        check(c, yy, label=f"{name} swiglu={swiglu} w16={w16} resid={resid}")


BWD_OPS = ["t", "t_acc", "at", "at_acc", "at_swiglu", "at_acc_swiglu"]


@pytest.mark.parametrize("cfg", [None] + list(range(24)))
def test_backward_every_config(cfg):
    """matmul_t: dX [292 x 68] over a 292-long contraction; matmul_at: dW
    [68 x 292] over 292 rows; with and without accumulation, and with the
    SwiGLU activation recomputed."""
    from tiled_dense_gemm_matmul_amd import binding
    if cfg is not None and cfg >= binding.bwd_num_configs():
        pytest.skip("no such configuration")
    M, K, N = 292, 68, 292
    name = "library's choice" if cfg is None else binding.bwd_config_name(cfg)
    for op in BWD_OPS:
        say(f"guards backward {name} {op} M={M} K={K} N={N}")
        acc = "acc" in op
        c = inputs.backward_case(40 + BWD_OPS.index(op), M, K, N, swiglu="swiglu" in op, acc=acc, gate_scale=3.0)
        dY = poisoned(c["dY"])
        if op.startswith("t"):
            out = Banded((M, K), c["dX0"] if acc else None)
            binding.matmul_t(dY, poisoned(c["W"]), out=out.view, acc=acc, config=cfg)
        elif "swiglu" in op:
            out = Banded((K, N), c["dW0"] if acc else None)
            binding.matmul_at_swiglu_a(poisoned(c["G"]), poisoned(c["U"]), dY, out=out.view, acc=acc, config=cfg)
        else:
            out = Banded((K, N), c["dW0"] if acc else None)
            binding.matmul_at(poisoned(c["X"]), dY, out=out.view, acc=acc, config=cfg)
        yy = out.result(f"{name} {op}")
        assert np.all(np.isfinite(yy)), f"{name} {op}: NaN from outside an input"
        check_bwd(c, op, yy, label=name)


@pytest.mark.parametrize("cfg", [None] + list(range(24)))
def test_fused_swiglu_backward_every_config(cfg):
    """dGATE, dUP from dH = dY W^T in matmul_t's epilogue: GATE and UP read
    there (poisoned neighbours), both gradients banded."""
    from tiled_dense_gemm_matmul_amd import binding
    if cfg is not None and cfg >= binding.bwd_num_configs():
        pytest.skip("no such configuration")
    M, K, N = 130, 68, 292
    name = "library's choice" if cfg is None else binding.bwd_config_name(cfg)
    say(f"guards fused SwiGLU backward {name} M={M} K={K} N={N}")
    c, G, U = fused_case(9, M, K, N)
    dg, du = Banded((M, K)), Banded((M, K))
    binding.matmul_t_swiglu_backward(poisoned(c["dY"]), poisoned(c["W"]), poisoned(G), poisoned(U),
                                     grad_gate=dg.view, grad_up=du.view, config=cfg)
    rg, ru, bg, bu = fused_ref(c, G, U)
    check_fused(dg.result(name), rg, bg, f"dGATE {name}")
    check_fused(du.result(name), ru, bu, f"dUP {name}")


@pytest.mark.parametrize("S,V", [(37, 1003), (33, 4096), (11, 8196), (7, 20000), (5, 70001)])
def test_loss_kernels(S, V):
    """cross_entropy rewrites the logits in place: they sit inside sentinel
    bands that must neither be read (the losses would change) nor written;
    the targets' neighbours are 0, the losses are banded; sum_losses reads
    poisoned losses into a banded total."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    say(f"guards loss S={S} V={V}")
    lc = inputs.loss_case(S * 7 + V, S, V, ignore_every=5)
    logits = Banded((S, V), lc["logits"], sentinel=50.0)
    tbuf = torch.zeros((2 * PAD + S,), dtype=torch.int32, device=device())
    tbuf[PAD:PAD + S] = torch.from_numpy(lc["targets"].astype(np.int32)).to(device())
    targets = tbuf[PAD:PAD + S]
    losses = Banded((S,))
    valid = int(np.count_nonzero(lc["targets"] < V))
    inv = 1.0 / valid
    binding.cross_entropy(logits.view, targets, alpha=0.1, beta=1e-4, inv_norm=inv, losses=losses.view)
    lref, gref, mag = OL.cross_entropy(lc["logits"], lc["targets"], 0.1, 1e-4, inv)
    res = oracle.compare(losses.result("losses"), lref, mag["loss"], OL.TOL_LOSS)
    assert res["fails"] == 0, res
    res = oracle.compare(logits.result("dlogits"), gref, mag["dlogits"], OL.TOL_DLOGITS)
    assert res["fails"] == 0, res
    total = Banded((1,))
    binding.sum_losses(poisoned(lref.astype(np.float32)), out=total.view)
    t = total.result("sum_losses")
    assert np.isfinite(t).all()
    assert abs(float(t[0]) - OL.sum_losses(lref.astype(np.float32))) <= 1e-5 * float(np.abs(lref).sum()) + 1e-6


@pytest.mark.parametrize("n", [4097, 100003, 512 * 3072])
def test_activation_kernels(n):
    from tiled_dense_gemm_matmul_amd import binding
    say(f"guards activation n={n}")
    c = inputs.activation_case(n % 997 + 3, n)
    g, x, u = poisoned(c["g"]), poisoned(c["gate"]), poisoned(c["up"])
    dg, du = Banded((n,)), Banded((n,))
    binding.ffn_swiglu_backward(g, x, u, grad_gate=dg.view, grad_up=du.view)
    rdg, rdu, sg, su = OA.ffn_swiglu_backward(c["g"], c["gate"], c["up"])
    assert oracle.compare(dg.result("grad_gate"), rdg, sg, OA.TOL)["fails"] == 0
    assert oracle.compare(du.result("grad_up"), rdu, su, OA.TOL)["fails"] == 0
    dp = Banded((n,))
    binding.ffn_gelu_backward(g, x, grad_pre=dp.view)
    rdp, sp = OA.ffn_gelu_backward(c["g"], c["gate"])
    assert oracle.compare(dp.result("grad_pre"), rdp, sp, OA.TOL)["fails"] == 0
    y, keep = Banded((n,), c["gate"], sentinel=3.0), Banded((n,))
    binding.gelu_inplace(y.view, pre_gelu=keep.view)
    ry, sy = OA.gelu_inplace(c["gate"])
    assert oracle.compare(y.result("gelu"), ry, sy, OA.TOL)["fails"] == 0
    assert np.array_equal(keep.result("pre_gelu"), c["gate"])
