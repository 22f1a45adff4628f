"""Python binding over libgemmfwd.so (the C ABI declared in include/gemm_fwd.h).

Argument marshalling only: shapes, dtypes and devices are checked, pointers and
the current HIP stream are passed through, and every step of the computation
runs in the library's HIP kernels.  torch provides device memory and streams.
The library must be built (``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

GEMM_FLAG_W_F16 = 0x1
GEMM_FLAG_ACC = 0x2
GEMM_W_F32 = 0
GEMM_W_F16 = 1

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemmfwd.so")
_lib = None

EXPORTED = (
    "gemm_fwd", "gemm_fwd_swiglu", "gemm_fwd_ex", "gemm_fwd_swiglu_ex", "gemm_fwd_workspace_bytes",
    "gemm_fwd_swiglu_noalloc",
    "gemm_num_configs", "gemm_config_name", "gemm_select_config", "gemm_status_string",
    "gemm_matmul_t", "gemm_matmul_at", "gemm_matmul_at_swiglu_a", "gemm_matmul_t_ex", "gemm_matmul_at_ex",
    "gemm_matmul_at_swiglu_a_ex", "gemm_bwd_num_configs", "gemm_bwd_config_name", "gemm_bwd_select_config",
    "gemm_bwd_workspace_bytes", "gemm_matmul_t_swiglu_bwd", "gemm_matmul_t_swiglu_bwd_ex",
    "loss_cross_entropy", "loss_sum_losses", "act_ffn_swiglu_backward", "act_ffn_gelu_backward",
    "act_gelu_inplace", "gemm_timing_event_create", "gemm_timing_event_record", "gemm_timing_elapsed_ms",
    "gemm_timing_event_destroy",
)


class GemmOpts(ctypes.Structure):
    """struct gemm_opts of include/gemm_fwd.h."""
    _fields_ = [("config", ctypes.c_int64), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64),
                ("start_event", ctypes.c_void_p), ("stop_event", ctypes.c_void_p)]


def opts(config=-1, workspace=None, workspace_bytes=0, start=None, stop=None):
    """A gemm_opts passed by reference (ctypes.byref) to the _ex entry points."""
    return ctypes.byref(GemmOpts(-1 if config is None else int(config), workspace, int(workspace_bytes), start, stop))


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


SYNC_CHECK_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemmfwd_sync.so")
_sync_lib = None


def load_library():
    """Load libgemmfwd.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        _lib = _open(_LIB_PATH)
    return _lib


def load_sync_check_library():
    """The verification build (same C ABI; see the race-check tests)."""
    global _sync_lib
    if _sync_lib is None:
        _sync_lib = _open(SYNC_CHECK_LIB_PATH)
    return _sync_lib


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    p, i64, u32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
    lib.gemm_fwd.argtypes = [p, p, p, p, i64, i64, i64, u32, p]
    lib.gemm_fwd.restype = c_int
    lib.gemm_fwd_swiglu.argtypes = [p, p, p, p, p, i64, i64, i64, c_int, p]
    lib.gemm_fwd_swiglu.restype = c_int
    o = ctypes.c_void_p  # const gemm_opts * (ctypes.byref or None)
    lib.gemm_fwd_ex.argtypes = [p, p, p, p, i64, i64, i64, u32, o, p]
    lib.gemm_fwd_ex.restype = c_int
    lib.gemm_fwd_swiglu_ex.argtypes = [p, p, p, p, p, i64, i64, i64, c_int, o, p]
    lib.gemm_fwd_swiglu_ex.restype = c_int
    lib.gemm_fwd_swiglu_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, c_int, p]
    lib.gemm_fwd_swiglu_noalloc.restype = c_int
    lib.gemm_fwd_workspace_bytes.argtypes = [i64, i64, i64, c_int, u32, c_int]
    lib.gemm_fwd_workspace_bytes.restype = i64
    lib.gemm_num_configs.argtypes = []
    lib.gemm_num_configs.restype = c_int
    lib.gemm_config_name.argtypes = [c_int]
    lib.gemm_config_name.restype = ctypes.c_char_p
    lib.gemm_select_config.argtypes = [i64, i64, i64, c_int, c_int, c_int]
    lib.gemm_select_config.restype = c_int
    lib.gemm_status_string.argtypes = [c_int]
    lib.gemm_status_string.restype = ctypes.c_char_p
    for name, n_in in (("gemm_matmul_t", 2), ("gemm_matmul_at", 2), ("gemm_matmul_at_swiglu_a", 3)):
        getattr(lib, name).argtypes = [p] * (n_in + 1) + [i64, i64, i64, u32, p]
        getattr(lib, name).restype = c_int
        getattr(lib, name + "_ex").argtypes = [p] * (n_in + 1) + [i64, i64, i64, u32, o, p]
        getattr(lib, name + "_ex").restype = c_int
    lib.gemm_matmul_t_swiglu_bwd.argtypes = [p] * 6 + [i64, i64, i64, p]
    lib.gemm_matmul_t_swiglu_bwd.restype = c_int
    lib.gemm_matmul_t_swiglu_bwd_ex.argtypes = [p] * 6 + [i64, i64, i64, o, p]
    lib.gemm_matmul_t_swiglu_bwd_ex.restype = c_int
    lib.gemm_bwd_workspace_bytes.argtypes = [c_int, i64, i64, i64, c_int, c_int]
    lib.gemm_bwd_workspace_bytes.restype = i64
    lib.gemm_bwd_num_configs.argtypes = []
    lib.gemm_bwd_num_configs.restype = c_int
    lib.gemm_bwd_config_name.argtypes = [c_int]
    lib.gemm_bwd_config_name.restype = ctypes.c_char_p
    lib.gemm_bwd_select_config.argtypes = [c_int, i64, i64, i64, c_int, c_int]
    lib.gemm_bwd_select_config.restype = c_int
    f32 = ctypes.c_float
    lib.loss_cross_entropy.argtypes = [p, p, p, i64, i64, f32, f32, f32, p]
    lib.loss_cross_entropy.restype = c_int
    lib.loss_sum_losses.argtypes = [p, p, i64, p]
    lib.loss_sum_losses.restype = c_int
    lib.act_ffn_swiglu_backward.argtypes = [p, p, p, p, p, i64, p]
    lib.act_ffn_swiglu_backward.restype = c_int
    lib.act_ffn_gelu_backward.argtypes = [p, p, p, i64, p]
    lib.act_ffn_gelu_backward.restype = c_int
    lib.act_gelu_inplace.argtypes = [p, p, i64, p]
    lib.act_gelu_inplace.restype = c_int
    lib.gemm_timing_event_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.gemm_timing_event_create.restype = c_int
    lib.gemm_timing_event_record.argtypes = [p, p]
    lib.gemm_timing_event_record.restype = c_int
    lib.gemm_timing_elapsed_ms.argtypes = [p, p, ctypes.POINTER(f32)]
    lib.gemm_timing_elapsed_ms.restype = c_int
    lib.gemm_timing_event_destroy.argtypes = [p]
    lib.gemm_timing_event_destroy.restype = c_int
    return lib


class TimingEvent:
    """A timing event of the library (gemm_timing_event_create: no
    system-scope cache writeback when it is recorded) for the start_event /
    stop_event of gemm_opts; `handle` is what opts() takes."""

    def __init__(self):
        h = ctypes.c_void_p()
        st = load_library().gemm_timing_event_create(ctypes.byref(h))
        if st != 0:
            raise GemmError(st, "gemm_timing_event_create")
        self.handle = h.value

    def record(self, stream=None) -> None:
        """Record the event on `stream` (a torch stream or a raw handle;
        None: torch's current stream) as a marker between launches."""
        if stream is None:
            stream = torch.cuda.current_stream()
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        st = load_library().gemm_timing_event_record(self.handle, handle)
        if st != 0:
            raise GemmError(st, "gemm_timing_event_record")

    def elapsed_ms(self, stop: "TimingEvent") -> float:
        """Milliseconds from this event to `stop` (both recorded and complete)."""
        ms = ctypes.c_float()
        st = load_library().gemm_timing_elapsed_ms(self.handle, stop.handle, ctypes.byref(ms))
        if st != 0:
            raise GemmError(st, "gemm_timing_elapsed_ms")
        return ms.value

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.gemm_timing_event_destroy(self.handle)
            self.handle = None


def status_string(status: int) -> str:
    return load_library().gemm_status_string(int(status)).decode()


def num_configs() -> int:
    return load_library().gemm_num_configs()


def config_name(config: int):
    name = load_library().gemm_config_name(int(config))
    return None if name is None else name.decode()


def config_takes_w16(config: int) -> bool:
    """Whether forward configuration `config` has binary16-W kernels: the
    tiles that load W straight into the compute waves' registers (names
    ending in _wrN) are fp32-only, and the library refuses them binary16 W."""
    return "_wr" not in config_name(config)


def bwd_num_configs() -> int:
    return load_library().gemm_bwd_num_configs()


def bwd_config_name(config: int):
    name = load_library().gemm_bwd_config_name(int(config))
    return None if name is None else name.decode()


def bwd_kernel_config(op, M, K, N, swiglu=False, workspace=True) -> str:
    """Name of the configuration the library picks for a backward product
    (op "matmul_t" or "matmul_at"; M, K, N the forward's names), with or
    without a workspace."""
    code = {"matmul_t": 1, "matmul_at": 2}[op]
    return bwd_config_name(load_library().gemm_bwd_select_config(code, M, K, N, int(swiglu), int(workspace)))


def kernel_config(M, K, N, swiglu=False, w16=False, workspace=True) -> str:
    """Name of the tile configuration the library picks for a shape, with or
    without a workspace."""
    return config_name(load_library().gemm_select_config(M, K, N, int(swiglu), int(w16), int(workspace)))


# --- split-K workspaces ---
#
# The library holds no device memory: split-K partial tiles go to a
# workspace the caller provides.  The tensor-level calls below keep one
# zero-filled torch buffer per (device, stream), grown on demand; the library
# leaves a workspace zeroed after every call, and calls on one stream are
# ordered, so the buffer is reused as it is.  Calls on different streams get
# different buffers.

_workspaces = {}


def workspace(device, stream, nbytes):
    """(pointer, size) of the zero-filled workspace for `stream` on `device`,
    at least nbytes long; (None, 0) when nbytes is 0."""
    if nbytes <= 0:
        return None, 0
    key = (device.index, int(stream.cuda_stream))
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(stream):
            # rounded up to a MiB: a few sizes serve every shape
            buf = torch.zeros(((nbytes + (1 << 20) - 1) >> 20) << 20, dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf.data_ptr(), buf.numel()


def _fwd_workspace(M, K, N, swiglu, w16, device, config):
    nbytes = load_library().gemm_fwd_workspace_bytes(M, K, N, int(swiglu), GEMM_FLAG_W_F16 if w16 else 0,
                                                     -1 if config is None else int(config))
    if nbytes < 0:
        raise GemmError(-2, "gemm_fwd_workspace_bytes")
    return workspace(device, torch.cuda.current_stream(device), nbytes)


# --- raw pointer-level calls (same names and argument order as the C ABI) ---

def gemm_fwd(X, W, R, Y, M, K, N, flags, stream) -> int:
    return load_library().gemm_fwd(X, W, R, Y, M, K, N, flags, stream)


def gemm_fwd_swiglu(G, U, W, R, Y, M, K, N, w_dtype, stream) -> int:
    return load_library().gemm_fwd_swiglu(G, U, W, R, Y, M, K, N, w_dtype, stream)


def gemm_fwd_ex(X, W, R, Y, M, K, N, flags, options, stream) -> int:
    return load_library().gemm_fwd_ex(X, W, R, Y, M, K, N, flags, options, stream)


def gemm_fwd_swiglu_ex(G, U, W, R, Y, M, K, N, w_dtype, options, stream) -> int:
    return load_library().gemm_fwd_swiglu_ex(G, U, W, R, Y, M, K, N, w_dtype, options, stream)


# --- tensor-level API ---

def _check_act(t, name, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_w(W, K, device):
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise TypeError("W must be a 2-D torch.Tensor [K, N]")
    if W.device != device:
        raise ValueError(f"W must live on {device}, got {W.device}")
    if W.dtype not in (torch.float32, torch.float16):
        raise TypeError(f"W must be float32 or float16, got {W.dtype}")
    if not W.is_contiguous():
        raise ValueError("W must be contiguous (row-major [K, N])")
    if W.shape[0] != K:
        raise ValueError(f"W has {W.shape[0]} rows, expected K={K}")
    return W.shape[1]


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def matmul(X, W, R=None, out=None, config=None, use_workspace=True):
    """Y = X @ W (+ R).  X [M, K] f32, W [K, N] f32 or f16, R [M, N] f32 or None.
    config: a configuration index (None: the library's choice).  use_workspace:
    give the library the stream's split-K workspace (False: the plain
    gemm_fwd behaviour, no split-K)."""
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise TypeError("X must be a 2-D torch.Tensor [M, K]")
    M, K = X.shape
    device = X.device
    _check_act(X, "X", (M, K), device)
    N = _check_w(W, K, device)
    if R is not None:
        _check_act(R, "R", (M, N), device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=device)
    else:
        _check_act(out, "out", (M, N), device)
    w16 = W.dtype == torch.float16
    flags = GEMM_FLAG_W_F16 if w16 else 0
    ws, wsb = _fwd_workspace(M, K, N, False, w16, device, config) if use_workspace else (None, 0)
    st = gemm_fwd_ex(X.data_ptr(), W.data_ptr(), None if R is None else R.data_ptr(), out.data_ptr(),
                     M, K, N, flags, opts(config, ws, wsb), _stream(device))
    if st != 0:
        raise GemmError(st, "gemm_fwd_ex")
    return out


def matmul_residual(X, W, R, out=None, config=None, use_workspace=True):
    """Y = X @ W + R."""
    if R is None:
        raise ValueError("matmul_residual needs R")
    return matmul(X, W, R, out=out, config=config, use_workspace=use_workspace)


def matmul_residual_swiglu_a(G, U, W, R, out=None, config=None, use_workspace=True):
    """Y = (silu(G) * U) @ W + R, the SwiGLU combine fused into the A load
    (config and use_workspace as for matmul)."""
    if not isinstance(G, torch.Tensor) or G.dim() != 2:
        raise TypeError("G must be a 2-D torch.Tensor [M, K]")
    M, K = G.shape
    device = G.device
    _check_act(G, "G", (M, K), device)
    _check_act(U, "U", (M, K), device)
    N = _check_w(W, K, device)
    _check_act(R, "R", (M, N), device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=device)
    else:
        _check_act(out, "out", (M, N), device)
    w16 = W.dtype == torch.float16
    w_dtype = GEMM_W_F16 if w16 else GEMM_W_F32
    ws, wsb = _fwd_workspace(M, K, N, True, w16, device, config) if use_workspace else (None, 0)
    st = gemm_fwd_swiglu_ex(G.data_ptr(), U.data_ptr(), W.data_ptr(), R.data_ptr(), out.data_ptr(),
                            M, K, N, w_dtype, opts(config, ws, wsb), _stream(device))
    if st != 0:
        raise GemmError(st, "gemm_fwd_swiglu_ex")
    return out


# --- backward linear family (matmul_t, matmul_at and their _acc / _swiglu_a forms) ---

def _bwd_workspace(op, M, K, N, swiglu, device, config):
    nbytes = load_library().gemm_bwd_workspace_bytes(op, M, K, N, int(swiglu), -1 if config is None else int(config))
    if nbytes < 0:
        raise GemmError(-2, "gemm_bwd_workspace_bytes")
    return workspace(device, torch.cuda.current_stream(device), nbytes)


def _bwd_call(name, ptrs, M, K, N, acc, device, config, use_workspace=True):
    lib = load_library()
    flags = GEMM_FLAG_ACC if acc else 0
    op = 1 if name == "gemm_matmul_t" else 2
    ws, wsb = (_bwd_workspace(op, M, K, N, name.endswith("swiglu_a"), device, config) if use_workspace
               else (None, 0))
    st = getattr(lib, name + "_ex")(*ptrs, M, K, N, flags, opts(config, ws, wsb), _stream(device))
    if st != 0:
        raise GemmError(st, name)


def _out(out, shape, device, acc):
    if out is None:
        if acc:
            raise ValueError("accumulation needs the output tensor")
        return torch.empty(shape, dtype=torch.float32, device=device)
    _check_act(out, "out", shape, device)
    return out


def matmul_t(dY, W, out=None, acc=False, config=None, use_workspace=True):
    """dX = dY @ W^T (matmul_t), or out += dY @ W^T with acc=True (matmul_t_acc).
    dY [M, N] f32, W [K, N] f32 (the forward's weight); dX [M, K]."""
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise TypeError("dY must be a 2-D torch.Tensor [M, N]")
    M, N = dY.shape
    device = dY.device
    _check_act(dY, "dY", (M, N), device)
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise TypeError("W must be a 2-D torch.Tensor [K, N]")
    K = W.shape[0]
    _check_act(W, "W", (K, N), device)
    out = _out(out, (M, K), device, acc)
    _bwd_call("gemm_matmul_t", (dY.data_ptr(), W.data_ptr(), out.data_ptr()), M, K, N, acc, device, config,
              use_workspace)
    return out


def matmul_at(X, dY, out=None, acc=False, config=None, use_workspace=True):
    """dW = X^T @ dY (matmul_at), or out += X^T @ dY with acc=True (matmul_at_acc).
    X [M, K] f32, dY [M, N] f32; dW [K, N]."""
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise TypeError("X must be a 2-D torch.Tensor [M, K]")
    M, K = X.shape
    device = X.device
    _check_act(X, "X", (M, K), device)
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise TypeError("dY must be a 2-D torch.Tensor [M, N]")
    N = dY.shape[1]
    _check_act(dY, "dY", (M, N), device)
    out = _out(out, (K, N), device, acc)
    _bwd_call("gemm_matmul_at", (X.data_ptr(), dY.data_ptr(), out.data_ptr()), M, K, N, acc, device, config,
              use_workspace)
    return out


def matmul_at_swiglu_a(G, U, dY, out=None, acc=False, config=None, use_workspace=True):
    """dW = (silu(G) * U)^T @ dY (matmul_at_swiglu_a), or out += ... with acc=True
    (matmul_at_acc_swiglu_a); the combine is recomputed as A is staged.
    G, U [M, K] f32, dY [M, N] f32; dW [K, N]."""
    if not isinstance(G, torch.Tensor) or G.dim() != 2:
        raise TypeError("G must be a 2-D torch.Tensor [M, K]")
    M, K = G.shape
    device = G.device
    _check_act(G, "G", (M, K), device)
    _check_act(U, "U", (M, K), device)
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise TypeError("dY must be a 2-D torch.Tensor [M, N]")
    N = dY.shape[1]
    _check_act(dY, "dY", (M, N), device)
    out = _out(out, (K, N), device, acc)
    _bwd_call("gemm_matmul_at_swiglu_a", (G.data_ptr(), U.data_ptr(), dY.data_ptr(), out.data_ptr()),
              M, K, N, acc, device, config, use_workspace)
    return out


def matmul_t_swiglu_backward(dY, W, G, U, grad_gate=None, grad_up=None, config=None):
    """The FFN down-projection's input gradient dH = dY @ W^T turned straight
    into the SwiGLU gradients (dH itself is never stored):
    grad_gate = nan_guard(dH * U * silu'(G)), grad_up = nan_guard(dH * silu(G)).
    dY [M, N], W [K, N] (the forward weight), G, U [M, K] f32.
    Returns (grad_gate, grad_up); either may be given as G or U to overwrite it."""
    if not isinstance(dY, torch.Tensor) or dY.dim() != 2:
        raise TypeError("dY must be a 2-D torch.Tensor [M, N]")
    M, N = dY.shape
    device = dY.device
    _check_act(dY, "dY", (M, N), device)
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise TypeError("W must be a 2-D torch.Tensor [K, N]")
    K = W.shape[0]
    _check_act(W, "W", (K, N), device)
    _check_act(G, "G", (M, K), device)
    _check_act(U, "U", (M, K), device)
    grad_gate = torch.empty((M, K), dtype=torch.float32, device=device) if grad_gate is None else grad_gate
    grad_up = torch.empty((M, K), dtype=torch.float32, device=device) if grad_up is None else grad_up
    _check_act(grad_gate, "grad_gate", (M, K), device)
    _check_act(grad_up, "grad_up", (M, K), device)
    lib = load_library()
    ptrs = (dY.data_ptr(), W.data_ptr(), G.data_ptr(), U.data_ptr(), grad_gate.data_ptr(), grad_up.data_ptr())
    ws, wsb = _bwd_workspace(1, M, K, N, False, device, config)
    st = lib.gemm_matmul_t_swiglu_bwd_ex(*ptrs, M, K, N, opts(config, ws, wsb), _stream(device))
    if st != 0:
        raise GemmError(st, "gemm_matmul_t_swiglu_bwd_ex")
    return grad_gate, grad_up


# --- fused loss (include/loss.h) ---

def cross_entropy(logits, targets, alpha=0.0, beta=0.0, inv_norm=None, losses=None):
    """cross_entropy: per-row losses, and the gradient written over `logits`
    in place.  logits [S, V] f32, targets [S] int32/int64 (values >= V, or
    negative, mark ignored rows); inv_norm defaults to 1 / (number of rows
    with a target in [0, V)), which reads that count back to the host.
    Returns the losses [S] f32 tensor."""
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise TypeError("logits must be a 2-D torch.Tensor [S, V]")
    S, V = logits.shape
    device = logits.device
    _check_act(logits, "logits", (S, V), device)
    if not isinstance(targets, torch.Tensor) or tuple(targets.shape) != (S,) or targets.device != device:
        raise ValueError(f"targets must be a [{S}] tensor on {device}")
    if targets.dtype not in (torch.int32, torch.int64):
        raise TypeError("targets must be int32 or int64")
    # the kernel reads targets as uint32: a negative value reads as >= V and
    # marks an ignored row, like any other out-of-range target
    t32 = targets if targets.dtype == torch.int32 and targets.is_contiguous() else targets.to(torch.int32).contiguous()
    if inv_norm is None:
        valid = int(((targets >= 0) & (targets < V)).sum().item())
        inv_norm = 1.0 / valid if valid else 0.0
    if losses is None:
        losses = torch.empty((S,), dtype=torch.float32, device=device)
    else:
        _check_act(losses, "losses", (S,), device)
    st = load_library().loss_cross_entropy(logits.data_ptr(), t32.data_ptr(), losses.data_ptr(), S, V,
                                           float(alpha), float(beta), float(inv_norm), _stream(device))
    if st != 0:
        raise GemmError(st, "loss_cross_entropy")
    return losses


def sum_losses(losses, out=None):
    """sum_losses: the scalar total of the per-row losses, as a [1] tensor."""
    if not isinstance(losses, torch.Tensor) or losses.dim() != 1:
        raise TypeError("losses must be a 1-D torch.Tensor")
    device = losses.device
    _check_act(losses, "losses", tuple(losses.shape), device)
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=device)
    else:
        _check_act(out, "out", (1,), device)
    st = load_library().loss_sum_losses(losses.data_ptr(), out.data_ptr(), losses.shape[0], _stream(device))
    if st != 0:
        raise GemmError(st, "loss_sum_losses")
    return out


# --- FFN activation kernels (include/activation.h) ---

def _same_shape(name, t, ref):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 torch.Tensor")
    if t.device != ref.device or t.shape != ref.shape:
        raise ValueError(f"{name} must have shape {tuple(ref.shape)} on {ref.device}")


def ffn_swiglu_backward(grad_hidden, gate, up, grad_gate=None, grad_up=None):
    """grad_gate = nan_guard(g * up * silu'(gate)), grad_up = nan_guard(g * silu(gate)),
    element-wise over tensors of one shape.  Returns (grad_gate, grad_up)."""
    _same_shape("grad_hidden", grad_hidden, grad_hidden)
    _same_shape("gate", gate, grad_hidden)
    _same_shape("up", up, grad_hidden)
    grad_gate = torch.empty_like(gate) if grad_gate is None else grad_gate
    grad_up = torch.empty_like(up) if grad_up is None else grad_up
    _same_shape("grad_gate", grad_gate, grad_hidden)
    _same_shape("grad_up", grad_up, grad_hidden)
    st = load_library().act_ffn_swiglu_backward(grad_hidden.data_ptr(), gate.data_ptr(), up.data_ptr(),
                                                grad_gate.data_ptr(), grad_up.data_ptr(), grad_hidden.numel(),
                                                _stream(grad_hidden.device))
    if st != 0:
        raise GemmError(st, "act_ffn_swiglu_backward")
    return grad_gate, grad_up


def ffn_gelu_backward(grad_hidden, pre_gelu, grad_pre=None):
    """grad_pre = nan_guard(g * gelu'(pre_gelu)), element-wise."""
    _same_shape("grad_hidden", grad_hidden, grad_hidden)
    _same_shape("pre_gelu", pre_gelu, grad_hidden)
    grad_pre = torch.empty_like(pre_gelu) if grad_pre is None else grad_pre
    _same_shape("grad_pre", grad_pre, grad_hidden)
    st = load_library().act_ffn_gelu_backward(grad_hidden.data_ptr(), pre_gelu.data_ptr(), grad_pre.data_ptr(),
                                              grad_hidden.numel(), _stream(grad_hidden.device))
    if st != 0:
        raise GemmError(st, "act_ffn_gelu_backward")
    return grad_pre


def gelu_inplace(x, pre_gelu=None):
    """x = gelu(x) in place (tanh approximation); pre_gelu, if given, receives
    the input values.  Returns x."""
    _same_shape("x", x, x)
    if pre_gelu is not None:
        _same_shape("pre_gelu", pre_gelu, x)
    st = load_library().act_gelu_inplace(x.data_ptr(), None if pre_gelu is None else pre_gelu.data_ptr(), x.numel(),
                                         _stream(x.device))
    if st != 0:
        raise GemmError(st, "act_gelu_inplace")
    return x
