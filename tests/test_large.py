"""Operands past 4 GiB.

The ABI accepts M up to 2^31 - 1.  The kernels keep 32-bit offsets only
inside a tile (at most 256 rows of A or Y), a K-stage or a 16-row slice of
W, and address each tile, stage and slice from a 64-bit base, so an array
larger than 2^32 bytes must come out right in its last tiles as in its
first: with the library's choice and with a tile that loads W into
registers.  Here A (and UP) hold
2^20 + 37 rows of 1024 fp32 values, 4.3e9 bytes each; the weight gradient
contracts over those 2^20 + 37 rows.  Inputs are drawn on the device from
seeded generators (N(0, 1), weights scaled by 0.02).  The forward products
are compared with the oracle on sampled rows that include the last 300; the
weight gradient on every output."""
import numpy as np
import pytest

import oracle

from _gpu import device, say

pytestmark = pytest.mark.gpu

M_BIG = (1 << 20) + 37
K = 1024
N = 16


def _randn(shape, seed, scale=1.0):
    import torch
    g = torch.Generator(device=device()).manual_seed(seed)
    return torch.randn(shape, device=device(), generator=g) * scale


def _rows(M):
    rng = np.random.default_rng(5)
    return np.unique(np.concatenate([np.arange(0, 3), rng.choice(M - 300, 40, replace=False),
                                     np.arange(M - 300, M)])).astype(np.int64)


@pytest.mark.parametrize("tile", [None, "16x48x128_k4_sp4_pf3_il_dA_wr2"])
@pytest.mark.parametrize("swiglu", [False, True])
def test_forward_operands_past_4gib(swiglu, tile):
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    cfg = None if tile is None else next(i for i in range(binding.num_configs()) if binding.config_name(i) == tile)
    name = binding.kernel_config(M_BIG, K, N, swiglu=swiglu) if tile is None else tile
    say(f"forward swiglu={swiglu}: A {M_BIG}x{K} fp32 ({M_BIG * K * 4 / 2**30:.2f} GiB), N={N}, tile {name}")
    A = _randn((M_BIG, K), 11)
    U = _randn((M_BIG, K), 12) if swiglu else None
    W = _randn((K, N), 13, 0.02)
    R = _randn((M_BIG, N), 14)
    y = binding.matmul_residual_swiglu_a(A, U, W, R, config=cfg) if swiglu else binding.matmul(A, W, R, config=cfg)
    torch.cuda.synchronize()
    rows = _rows(M_BIG)
    idx = torch.from_numpy(rows).to(device())

    def pick(t):
        return np.ascontiguousarray(t.index_select(0, idx).cpu().numpy())
    ref, scale = oracle.gemm(pick(A), np.ascontiguousarray(W.cpu().numpy()), R=pick(R),
                             U=pick(U) if swiglu else None, want_scale=True)
    res = oracle.compare(pick(y), ref, scale, oracle.TOL_W32)
    say(f"  max err/tol {res['max_ratio']:.3g}, fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res


def test_weight_gradient_contraction_past_4gib():
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    say(f"matmul_at: X {M_BIG}x{K} fp32 ({M_BIG * K * 4 / 2**30:.2f} GiB), dY {M_BIG}x{N}, "
        f"tile {binding.bwd_kernel_config('matmul_at', M_BIG, K, N)}")
    X = _randn((M_BIG, K), 21)
    dY = _randn((M_BIG, N), 22)
    dW = binding.matmul_at(X, dY)
    torch.cuda.synchronize()
    x, dy = X.cpu().numpy(), dY.cpu().numpy()
    del X
    ref, scale = oracle.matmul_at(x, dy, want_scale=True)
    res = oracle.compare(dW.cpu().numpy(), ref, scale, oracle.TOL_W32)
    say(f"  max err/tol {res['max_ratio']:.3g}, fails {res['fails']} of {res['n']}")
    assert res["fails"] == 0, res
