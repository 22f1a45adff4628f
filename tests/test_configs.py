"""Every tile configuration compiled into the library, in every variant
(plain / SwiGLU A operand x fp32 / binary16 W x with / without residual), on
ragged shapes that leave partial tiles in M, N and K, against the oracle."""
import numpy as np
import pytest

from tiled_dense_gemm_matmul_amd import inputs

from _gpu import check, run, say

pytestmark = pytest.mark.gpu


def _num_configs():
    from tiled_dense_gemm_matmul_amd import binding
    return binding.num_configs()


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("w16", [False, True])
@pytest.mark.parametrize("resid", [False, True])
def test_all_configs_ragged(swiglu, w16, resid):
    from tiled_dense_gemm_matmul_amd import binding
    if swiglu and not resid:
        pytest.skip("the SwiGLU variant always has a residual")
    for (M, K, N) in [(77, 132, 100), (130, 68, 196), (33, 260, 52)]:
        case = inputs.random_case(M * 7 + K, M, K, N, swiglu=swiglu, w16=w16, residual=resid, gate_scale=3.0)
        for cfg in range(binding.num_configs()):
            if w16 and not binding.config_takes_w16(cfg):
                continue  # fp32-only tile (W in registers)
            say(f"config {binding.config_name(cfg)} M={M} K={K} N={N} swiglu={swiglu} w16={w16} resid={resid}")
            y = run(case, config=cfg).cpu().numpy()
            check(case, y, label=binding.config_name(cfg))
