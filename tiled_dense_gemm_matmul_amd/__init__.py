"""MI355X-native forward linear-layer GEMM family (gfx950, HIP + fp32 MFMA).

Public Python surface (a thin binding over the C-ABI library libgemmfwd.so):

    matmul(X, W, R=None, out=None)                      Y = X @ W (+ R)
    matmul_residual_swiglu_a(G, U, W, R, out=None)      Y = (silu(G) * U) @ W + R
    gemm_fwd(...), gemm_fwd_swiglu(...)                 raw C-ABI calls on pointers

W may be float32 or float16 ([K, N] row-major); activations are float32.
The binding (and with it torch and the HIP library) is loaded on first use, so
``tiled_dense_gemm_matmul_amd.inputs`` can be imported without either.
"""
_BINDING_NAMES = {
    "matmul", "matmul_residual", "matmul_residual_swiglu_a", "gemm_fwd", "gemm_fwd_swiglu",
    "status_string", "library_path", "load_library", "GemmError", "kernel_config",
    "num_configs", "config_name",
    "GEMM_FLAG_W_F16", "GEMM_W_F32", "GEMM_W_F16",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
