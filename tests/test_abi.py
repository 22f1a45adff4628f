"""The C-ABI boundary, on the CPU: the library loads, exports every function
that include/gemm_fwd.h declares, and rejects bad arguments synchronously with
the documented status codes before touching any device (all pointers here are
fake host addresses; no compute call reaches the GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_fwd.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z_0-9]+)\s*\(", text)))


def _status(name):
    m = re.search(r"#define\s+" + name + r"\s+\(?(-?\d+)\)?", _header_text())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    from tiled_dense_gemm_matmul_amd import binding
    return binding.load_library()


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert {"gemm_fwd", "gemm_fwd_swiglu", "gemm_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libgemmfwd.so does not export {n}"


def test_probe_library_exports_its_header():
    """The MFMA ceiling probe (measurement support for bench.py) exports what
    include/mfma_probe.h declares and rejects bad arguments without a launch."""
    path = os.path.join(ROOT, "tiled_dense_gemm_matmul_amd", "libmfmaprobe.so")
    if not os.path.exists(path):
        pytest.skip("libmfmaprobe.so not built")
    with open(os.path.join(ROOT, "include", "mfma_probe.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mfma_probe_[a-z_]+)\s*\(", text)))
    assert names == ["mfma_probe_flops", "mfma_probe_launch"]
    probe = ctypes.CDLL(path)
    for n in names:
        assert hasattr(probe, n)
    probe.mfma_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    probe.mfma_probe_flops.restype = ctypes.c_longlong
    assert probe.mfma_probe_launch(None, None, 1, 1, None) == -1
    assert probe.mfma_probe_launch(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 0, 1, None) == -1
    assert probe.mfma_probe_launch(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), 1, 0, None) == -1
    assert probe.mfma_probe_flops(256, 8192) == 256 * 4 * 8192 * 8 * 2048


def test_status_codes_match_header(lib):
    for name in ["GEMM_OK", "GEMM_ERR_NULL", "GEMM_ERR_SHAPE", "GEMM_ERR_ALIGN", "GEMM_ERR_DTYPE",
                 "GEMM_ERR_ALIAS", "GEMM_ERR_LAUNCH", "GEMM_ERR_CONFIG", "GEMM_ERR_WORKSPACE"]:
        code = _status(name)
        text = lib.gemm_status_string(code).decode()
        assert text and text != "unknown status", name
    assert lib.gemm_status_string(12345).decode() == "unknown status"


def test_config_table(lib):
    n = lib.gemm_num_configs()
    assert n >= 1
    names = [lib.gemm_config_name(i).decode() for i in range(n)]
    assert len(set(names)) == n
    assert lib.gemm_config_name(n) is None and lib.gemm_config_name(-1) is None
    # one shape per branch of the library's tile choice
    for shape in [(512, 768, 16384), (8192, 3072, 768), (1024, 768, 2048), (512, 768, 3072), (128, 768, 768),
                  (512, 3072, 768), (256, 4096, 768), (512, 768, 768), (8192, 768, 50304), (1, 4, 4)]:
        for sw in (0, 1):
            for w16 in (0, 1):
                for ws in (0, 1):
                    assert 0 <= lib.gemm_select_config(*shape, sw, w16, ws) < n

    def pick(M, K, N, sw, w16, ws=1):
        return lib.gemm_config_name(lib.gemm_select_config(M, K, N, sw, w16, ws)).decode()
    # the workload configurations (their tiles are the ones bench.py times)
    assert pick(128, 768, 768, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    assert pick(512, 768, 768, 0, 0) == "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert pick(512, 3072, 768, 1, 0) == "16x192x128_w1x4_sp4_pf3_il_ks2_wr4"
    assert pick(512, 768, 16384, 0, 1) == "128x128x32_w2x2_sp4_pf3_il_dA"
    assert pick(512, 768, 3072, 0, 1) == "128x48x32_w2x1_k2_sp4_pf3_il_dA"
    assert pick(8192, 3072, 768, 1, 1) == "64x384x32_w1x4_sp8_pf4_il"
    # a 128 x 64 grid filling under 70% of its rounds of two per CU
    assert pick(3072, 768, 1536, 0, 0) == "32x192x64_w1x4_sp4_pf3_il_dA_wr4"
    assert pick(6144, 768, 768, 0, 1) == "128x48x32_w2x1_k2_sp4_pf3_il_dA"
    assert pick(4608, 768, 1024, 0, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(3072, 768, 1536, 1, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(2304, 768, 2304, 0, 1) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert pick(2304, 768, 2304, 1, 1) == "64x64x64_w2x2_sp4_dAW"
    # a 64 x 64 grid filling under 70% of its rounds of two per CU
    assert pick(1536, 768, 1536, 0, 1) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert pick(1536, 768, 1536, 1, 0) == "32x192x64_w1x4_sp4_pf3_il_dA_wr4"
    assert pick(1536, 768, 1536, 1, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(2304, 768, 1152, 0, 1) == "128x48x32_w2x1_k2_sp4_pf3_il_dA"
    assert pick(448, 768, 6528, 0, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(8192, 768, 50304, 0, 1) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # small grids with fp32 W keep W in registers; f16 W stages it through LDS
    assert pick(128, 768, 768, 0, 1) == "16x48x128_k4_sp4_dAW"
    assert pick(512, 768, 768, 0, 1) == "32x48x128_k4_sp8_pf2_dAW"
    assert pick(512, 1024, 1024, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    assert pick(512, 1536, 768, 1, 0) == "16x96x128_w1x2_k2_sp8_pf2_il_wr4"
    assert pick(128, 3072, 768, 1, 0, ws=0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    # small outputs over a long contraction with fp32 W and a workspace: the
    # 16-row tile and two- or four-way K split of least estimated time
    assert pick(128, 3072, 768, 1, 0) == "16x96x128_w1x2_k2_sp4_pf3_il_ks4_dA_wr4"
    assert pick(64, 3072, 768, 1, 0) == "16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"
    assert pick(256, 3072, 768, 1, 0) == "16x192x128_w1x4_sp4_pf3_il_ks4_wr4"
    assert pick(128, 8192, 768, 0, 0) == "16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"
    assert pick(512, 8192, 512, 0, 0) == "16x48x128_k4_sp4_pf3_il_ks2_dA_wr2"
    assert pick(128, 8192, 768, 0, 0, ws=0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    # the same for binary16 W over the LDS-staged tiles
    assert pick(64, 3072, 768, 1, 1) == "16x48x128_k4_sp4_ks4_dAW"
    assert pick(128, 8192, 768, 0, 1) == "32x48x128_k4_sp8_pf2_ks4_dAW"
    assert pick(256, 3072, 768, 1, 1) == "32x96x128_w1x2_k2_sp8_pf3_il_ks4_cil_dAW"
    assert pick(128, 8192, 768, 0, 1, ws=0) == "16x48x128_k4_sp4_dAW"
    # few rows against a wide W: 16-row tiles instead of 128 x 64 / 64 x 64
    assert pick(16, 768, 50304, 0, 1) == "16x48x128_k4_sp4_dAW"
    assert pick(16, 768, 16384, 0, 0) == "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert pick(48, 768, 50304, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    assert pick(48, 4096, 16384, 0, 0) == "64x64x64_w2x2_sp4_ks2_dAW"
    assert pick(48, 4096, 16384, 0, 0, ws=0) == "64x64x64_w2x2_sp4_dAW"
    assert pick(64, 768, 50304, 0, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(65, 768, 50304, 0, 1) == "128x64x32_w2x2_sp4_pf3_il_dA"
    # 128 x 128 only where its grid fills 70% of its rounds
    assert pick(3072, 768, 3072, 0, 1) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert pick(4096, 768, 4096, 0, 1) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # one whole round of 64 x 64 tiles over a long contraction: K split in two
    # with a workspace (SwiGLU only while the split fits the library-held
    # scratch)
    assert pick(1024, 4096, 1024, 0, 0) == "64x64x64_w2x2_sp4_ks2_dAW"
    assert pick(1024, 4096, 1024, 0, 1) == "64x64x64_w2x2_sp4_ks2_dAW"
    assert pick(1024, 4096, 1024, 0, 0, ws=0) == "64x64x64_w2x2_sp4_dAW"
    assert pick(1024, 1024, 1024, 0, 0) == "64x64x64_w2x2_sp4_dAW"
    assert pick(1024, 4096, 1024, 1, 0) == "64x64x64_w2x2_sp4_dAW"
    # few columns: no tile more than twice as wide as the columns it covers
    assert pick(8192, 768, 48, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    assert pick(32768, 768, 64, 0, 0) == "64x64x64_w2x2_sp4_dAW"
    assert pick(32768, 768, 64, 1, 0) == "64x64x64_w2x2_sp4_dAW"
    assert pick(8192, 3072, 32, 1, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    # below 3072 of contraction only grids of at most half a round split
    assert pick(64, 2048, 768, 0, 0) == "16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"
    assert pick(128, 2048, 1024, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    assert pick(256, 768, 1024, 1, 0) == "16x96x128_w1x2_k2_sp8_pf2_il_wr4"
    # mid-size fp32 grids: 32 x 192 on whole rounds, else 16 x 96 / 16 x 48
    assert pick(2048, 768, 768, 0, 0) == "32x192x64_w1x4_sp4_pf3_il_dA_wr4"
    assert pick(2048, 768, 768, 0, 1) == "128x48x32_w2x1_k2_sp4_pf3_il_dA"
    assert pick(768, 768, 2048, 1, 0) == "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert pick(1000, 768, 772, 0, 0) == "16x48x128_k4_sp4_pf3_il_dA_wr2"
    # large SwiGLU grids with fp32 W: 32 x 384 (32 x 192 where N is far
    # from a multiple of 384), ahead of 128 x 128
    assert pick(8192, 3072, 768, 1, 0) == "32x384x64_w1x4_sp4_pf3_il_dA_wr2"
    assert pick(8192, 3072, 772, 1, 0) == "32x192x64_w1x4_sp4_pf3_il_dA_wr4"
    assert pick(8192, 1536, 1536, 1, 0) == "32x384x64_w1x4_sp4_pf3_il_dA_wr2"
    assert pick(8192, 1536, 1536, 1, 1) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # without a workspace the long-K small grid does not split K; with fp32 W
    # a plain A does not split it either way
    assert pick(512, 3072, 768, 1, 0, ws=0) == "16x96x128_w1x2_k2_sp8_pf2_il_wr4"
    assert pick(512, 3072, 768, 0, 0, ws=0) == "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert pick(512, 3072, 768, 0, 0) == "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert pick(512, 3072, 768, 1, 1) == "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW"
    assert pick(512, 3072, 768, 0, 1) == "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dAW"
    assert pick(512, 3072, 768, 1, 1, ws=0) == "16x96x128_w1x2_k2_sp8_pf3_il_cil_dW"
    # mid-size grids: 128 x 64 while it gives two tiles per CU, 64 x 64 when
    # it fills one whole round and 64 x 48 does not
    assert pick(512, 768, 8192, 0, 1) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert pick(512, 768, 2048, 0, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(512, 768, 4096, 0, 1) == "64x64x64_w2x2_sp4_dAW"
    assert pick(8192, 768, 768, 0, 0) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert pick(8192, 3072, 768, 0, 1) == "128x64x32_w2x2_sp4_pf3_il_dA"


def test_workspace_sizes(lib):
    """gemm_fwd_workspace_bytes / gemm_bwd_workspace_bytes: 0 for the
    configurations that do not split K; otherwise the 64 KiB counter block
    plus one M x N fp32 slot per split."""
    names = [lib.gemm_config_name(i).decode() for i in range(lib.gemm_num_configs())]
    CNT = 64 << 10
    # 512 x 3072 x 768 SwiGLU: 16 x 192 tiles (fp32 W) or 32 x 96 (f16 W), K
    # split in two
    assert lib.gemm_fwd_workspace_bytes(512, 3072, 768, 1, 0, -1) == CNT + 2 * 512 * 768 * 4
    assert lib.gemm_fwd_workspace_bytes(512, 3072, 768, 1, 1, -1) == CNT + 2 * 512 * 768 * 4
    assert lib.gemm_fwd_workspace_bytes(512, 3072, 768, 0, 0, -1) == 0
    assert lib.gemm_fwd_workspace_bytes(512, 768, 16384, 0, 1, -1) == 0
    assert lib.gemm_fwd_workspace_bytes(512, 3072, 768, 1, 0, names.index("128x128x32_w2x2_sp4_pf3_il_dA")) == 0
    ks8 = names.index("128x96x64_w2x2_sp8_ks8")
    assert lib.gemm_fwd_workspace_bytes(100, 64, 200, 0, 0, ks8) == CNT + 8 * 100 * 200 * 4
    # more output tiles than the counter block holds: refused
    assert lib.gemm_fwd_workspace_bytes(128 * 200, 64, 96 * 100, 0, 0, ks8) == -1
    assert lib.gemm_fwd_workspace_bytes(0, 64, 64, 0, 0, -1) == 0
    assert lib.gemm_fwd_workspace_bytes(-1, 64, 64, 0, 0, -1) == -1
    assert lib.gemm_fwd_workspace_bytes(64, 64, 64, 0, 2, -1) == -1
    assert lib.gemm_fwd_workspace_bytes(64, 64, 64, 0, 0, len(names)) == -1
    # the lm_head's input gradient: 128 x 96 tiles with the 16384-long
    # contraction split eight ways
    assert lib.gemm_bwd_workspace_bytes(1, 512, 768, 16384, 0, -1) == CNT + 8 * 512 * 768 * 4
    assert lib.gemm_bwd_workspace_bytes(2, 512, 768, 16384, 0, -1) == 0
    assert lib.gemm_bwd_workspace_bytes(3, 512, 768, 16384, 0, -1) == -1


# fake, well-aligned, non-overlapping host addresses
X, W, R, Y, U = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


WS = 0x60000000  # a fake workspace


def _opts(config=-1, ws=None, wsb=0):
    from tiled_dense_gemm_matmul_amd import binding
    return binding.opts(config, ws, wsb)


def fwd(lib, x=X, w=W, r=R, y=Y, M=64, K=64, N=64, flags=0, config=-1, ws=None, wsb=0):
    return lib.gemm_fwd_ex(x, w, r, y, M, K, N, flags, _opts(config, ws, wsb), None)


def sw(lib, g=X, u=U, w=W, r=R, y=Y, M=64, K=64, N=64, wd=0, config=-1, ws=None, wsb=0):
    return lib.gemm_fwd_swiglu_ex(g, u, w, r, y, M, K, N, wd, _opts(config, ws, wsb), None)


def test_null_pointers(lib):
    E = _status("GEMM_ERR_NULL")
    assert fwd(lib, x=None) == E
    assert fwd(lib, w=None) == E
    assert fwd(lib, y=None) == E
    assert sw(lib, u=None) == E
    assert sw(lib, r=None) == E  # the residual is required by the SwiGLU variant
    assert lib.gemm_fwd(None, W, None, Y, 4, 4, 4, 0, None) == E
    # arrays with no elements may have NULL storage (empty tensors)
    OK = _status("GEMM_OK")
    assert fwd(lib, x=None, y=None, M=0) == OK
    assert fwd(lib, w=None, y=None, N=0) == OK
    assert sw(lib, g=None, u=None, w=None, r=None, y=None, M=0, N=0) == OK


def test_shapes(lib):
    E = _status("GEMM_ERR_SHAPE")
    assert fwd(lib, K=6) == E
    assert fwd(lib, N=66) == E
    assert fwd(lib, M=-1) == E
    assert fwd(lib, K=-4) == E
    assert fwd(lib, N=1 << 31) == E
    assert fwd(lib, K=1 << 21) == E
    assert fwd(lib, N=1 << 21) == E
    assert fwd(lib, M=0, K=(1 << 21) - 4, N=(1 << 21) - 4) == _status("GEMM_OK")
    assert sw(lib, K=3074) == E


def test_alignment(lib):
    E = _status("GEMM_ERR_ALIGN")
    assert fwd(lib, x=X + 4) == E
    assert fwd(lib, y=Y + 8) == E
    assert fwd(lib, r=R + 12) == E
    assert fwd(lib, w=W + 8) == E                        # fp32 W needs 16 bytes
    assert fwd(lib, w=W + 8, flags=1, M=0) == _status("GEMM_OK")  # f16 W needs only 8 bytes
    assert fwd(lib, w=W + 4, flags=1) == E
    assert sw(lib, u=U + 4) == E


def test_dtype_and_config(lib):
    assert fwd(lib, flags=2) == _status("GEMM_ERR_DTYPE")
    assert sw(lib, wd=2) == _status("GEMM_ERR_DTYPE")
    assert sw(lib, wd=-1) == _status("GEMM_ERR_DTYPE")
    assert fwd(lib, config=lib.gemm_num_configs()) == _status("GEMM_ERR_CONFIG")
    assert fwd(lib, config=-2) == _status("GEMM_ERR_CONFIG")
    # tiles that keep W in registers are fp32-only: binary16 W is refused
    # before anything is enqueued, also for an empty output
    names = [lib.gemm_config_name(i).decode() for i in range(lib.gemm_num_configs())]
    wr = [i for i, n in enumerate(names) if "_wr" in n]
    assert len(wr) >= 4
    for c in wr:
        assert fwd(lib, flags=1, config=c) == _status("GEMM_ERR_CONFIG")
        assert fwd(lib, flags=1, config=c, r=None) == _status("GEMM_ERR_CONFIG")
        assert fwd(lib, flags=1, config=c, M=0) == _status("GEMM_ERR_CONFIG")
        assert sw(lib, wd=1, config=c) == _status("GEMM_ERR_CONFIG")


def test_workspace_validation(lib):
    """The workspace is checked before anything is enqueued: a split-K
    configuration forced without one, or with one that is too small, a
    pointer/size mismatch, a misaligned or overlapping workspace."""
    WSE, ALIGN, ALIAS = _status("GEMM_ERR_WORKSPACE"), _status("GEMM_ERR_ALIGN"), _status("GEMM_ERR_ALIAS")
    names = [lib.gemm_config_name(i).decode() for i in range(lib.gemm_num_configs())]
    ks2 = names.index("32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW")
    need = lib.gemm_fwd_workspace_bytes(64, 256, 64, 1, 0, ks2)
    assert need > 0
    assert sw(lib, K=256, config=ks2) == WSE
    assert sw(lib, K=256, config=ks2, ws=WS, wsb=need - 1) == WSE
    assert sw(lib, K=256, ws=None, wsb=64) == WSE
    assert sw(lib, K=256, ws=WS, wsb=-1) == WSE
    assert sw(lib, K=256, config=ks2, ws=WS + 16, wsb=need) == ALIGN
    assert sw(lib, K=256, config=ks2, ws=Y - 256, wsb=need) == ALIAS
    assert sw(lib, K=256, config=ks2, ws=X + 256, wsb=need) == ALIAS
    # a workspace adjacent to the arrays passes validation (checked on a
    # no-op shape)
    assert sw(lib, M=0, K=256, config=ks2, ws=WS, wsb=need) == _status("GEMM_OK")
    # backward: the same rules
    at = names  # (unused; the backward table has its own names)
    del at
    bwd = [lib.gemm_bwd_config_name(i).decode() for i in range(lib.gemm_bwd_num_configs())]
    ks8 = bwd.index("128x96x64_w2x2_sp8_pf3_il_ks8_cil_dA")
    t = lambda c=-1, ws=None, wsb=0: lib.gemm_matmul_t_ex(X, W, Y, 64, 64, 256, 0, _opts(c, ws, wsb), None)
    assert t(c=ks8) == WSE and t(ws=None, wsb=8) == WSE and t(c=ks8, ws=WS + 128, wsb=1 << 20) == ALIGN


def test_alias(lib):
    E = _status("GEMM_ERR_ALIAS")
    M = K = N = 64
    assert fwd(lib, r=Y) == E                          # in-place residual is rejected
    assert fwd(lib, x=Y + 16 * 4) == E                  # partial overlap
    assert fwd(lib, w=Y - 16 * 4) == E
    assert sw(lib, u=Y + M * N * 4 - 16) == E
    # adjacent, not overlapping: passes validation (checked on a no-op shape)
    assert fwd(lib, x=Y + M * N * 4, M=0) == _status("GEMM_OK")


def test_degenerate_shapes_are_noops(lib):
    OK = _status("GEMM_OK")
    assert fwd(lib, M=0) == OK
    assert fwd(lib, N=0) == OK
    assert sw(lib, M=0) == OK
    assert fwd(lib, M=0, K=0, N=0) == OK


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    from tiled_dense_gemm_matmul_amd import binding
    x = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        binding.matmul(x, x)


def test_backward_validation(lib):
    """matmul_t / matmul_at / matmul_at_swiglu_a reject bad arguments
    synchronously (fake host pointers; nothing reaches a device)."""
    NULL, SHAPE, ALIGN = _status("GEMM_ERR_NULL"), _status("GEMM_ERR_SHAPE"), _status("GEMM_ERR_ALIGN")
    DTYPE, ALIAS, CONFIG = _status("GEMM_ERR_DTYPE"), _status("GEMM_ERR_ALIAS"), _status("GEMM_ERR_CONFIG")
    ACC = 0x2
    t = lambda dy=X, w=W, y=Y, M=64, K=64, N=64, f=0, c=-1: lib.gemm_matmul_t_ex(dy, w, y, M, K, N, f, _opts(c),
                                                                                   None)
    at = lambda x=X, dy=W, y=Y, M=64, K=64, N=64, f=0, c=-1: lib.gemm_matmul_at_ex(x, dy, y, M, K, N, f, _opts(c),
                                                                                    None)
    ats = lambda g=X, u=U, dy=W, y=Y, M=64, K=64, N=64, f=0, c=-1: lib.gemm_matmul_at_swiglu_a_ex(
        g, u, dy, y, M, K, N, f, _opts(c), None)
    assert t(dy=None) == NULL and t(w=None) == NULL and t(y=None) == NULL
    assert at(x=None) == NULL and at(dy=None) == NULL and ats(u=None) == NULL
    assert t(K=6) == SHAPE and t(N=6) == SHAPE and at(K=10) == SHAPE and t(M=-1) == SHAPE
    assert t(dy=X + 4) == ALIGN and at(y=Y + 8) == ALIGN and ats(u=U + 4) == ALIGN
    assert t(f=0x1) == DTYPE and at(f=0x4) == DTYPE and ats(f=ACC | 0x1) == DTYPE
    assert t(y=X) == ALIAS and at(y=W + 64) == ALIAS and ats(y=U) == ALIAS
    assert t(c=lib.gemm_bwd_num_configs()) == CONFIG
    # M (the contraction of matmul_at) is unrestricted; empty outputs are no-ops
    assert t(M=0) == 0 and at(K=0) == 0 and at(N=0) == 0
    n = lib.gemm_bwd_num_configs()
    assert n >= 1 and all(lib.gemm_bwd_config_name(i) for i in range(n))
    assert lib.gemm_bwd_config_name(n) is None


def test_backward_selection(lib):
    n = lib.gemm_bwd_num_configs()
    for op in (1, 2):
        for shape in [(512, 768, 768), (512, 3072, 768), (512, 768, 3072), (512, 768, 16384), (8192, 3072, 768),
                      (1, 4, 4)]:
            for sw in ((0, 1) if op == 2 else (0,)):
                for ws in (0, 1):
                    assert 0 <= lib.gemm_bwd_select_config(op, *shape, sw, ws) < n, (op, shape, sw, ws)
    assert lib.gemm_bwd_select_config(0, 512, 768, 768, 0, 1) == -1
    assert lib.gemm_bwd_select_config(3, 512, 768, 768, 0, 1) == -1

    def name(op, *shape, ws=1):
        return lib.gemm_bwd_config_name(lib.gemm_bwd_select_config(op, *shape, 0, ws)).decode()
    # without a workspace the lm_head's input gradient does not split K
    assert name(1, 512, 768, 16384, ws=0) == "32x48x128_k4_sp8_pf2_dAW"
    # a transposed B over a long contraction onto a small grid: 32 x 48 or
    # 16 x 48 tiles, K split with a workspace (from 2048 on grids of at most
    # half a round, from 8192 beyond)
    assert name(1, 64, 768, 16384) == "32x48x128_k4_sp8_pf2_ks8_dAW"
    assert name(1, 128, 768, 16384) == "32x48x128_k4_sp8_pf2_ks4_dAW"
    assert name(1, 256, 768, 16384) == "32x48x128_k4_sp8_pf2_ks2_dAW"
    assert name(1, 256, 768, 16384, ws=0) == "16x48x128_k4_sp4_dAW"
    assert name(1, 256, 768, 3072) == "16x48x128_k4_sp4_dAW"
    # dW of the 768 x 768 projections: 384 tiles of 32 x 48 would take two
    # rounds on 256 CUs, 256 tiles of 48 x 48 take one
    assert name(2, 512, 768, 768) == "48x48x64_k4_sp4_pf3_dAW"
    # dW over the 512-token contraction whose 32 x 96 grid fills the CUs: dY
    # straight into registers
    assert name(2, 512, 768, 3072) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 512, 3072, 768) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(1, 512, 768, 16384) == "128x96x64_w2x2_sp8_pf3_il_ks8_cil_dA"
    assert name(1, 512, 768, 768) == "32x48x128_k4_sp8_pf2_dAW"
    assert name(1, 512, 3072, 768) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert name(1, 512, 768, 3072) == "16x48x128_k4_sp4_dAW"
    assert name(2, 512, 768, 16384) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # 16 x 512 tokens
    assert name(1, 8192, 768, 768) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert name(1, 8192, 768, 3072) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert name(1, 8192, 3072, 768) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # dW over 1024 tokens or more onto at most two rounds of 48 x 48 tiles:
    # those tiles, K split over two or four workgroups when there is a
    # workspace, as far as each keeps 512 of the contraction and the grid
    # stays within one workgroup per CU (two from 2048 tokens; a two-way
    # split up to four from 8192)
    assert name(2, 8192, 768, 768) == "48x48x64_k4_sp4_pf2_ks2_dAW"
    assert name(2, 16384, 768, 768) == "48x48x64_k4_sp4_pf2_ks2_dAW"
    assert name(2, 2048, 768, 768) == "48x48x64_k4_sp4_pf2_ks2_dAW"
    assert name(2, 8192, 768, 768, ws=0) == "48x48x64_k4_sp4_pf3_dAW"
    # a narrow dX over many tokens: no tile more than twice as wide as its
    # columns
    assert name(1, 32768, 64, 768) == "64x64x64_w2x2_sp4"
    # a transposed B where the rule takes 64 x 64: 64 x 48 where 48-wide
    # tiles cover the columns at least as fully
    assert name(1, 16384, 96, 3072) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert name(1, 4096, 768, 768) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert name(1, 8192, 256, 768) == "64x64x64_w2x2_sp4"
    # dX whose 128 x 128 grid spans more than one round of two per CU but
    # fills under 70% of its rounds: 128 x 64
    assert name(1, 3072, 3072, 768) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert name(1, 1536, 6144, 3072) == "128x64x32_w2x2_sp4_pf3_il_dA"
    assert name(1, 4096, 4096, 768) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # dX whose 128 x 64 or 64 x 64 grid fills under 60% of its rounds: 64 x 48
    assert name(1, 512, 4352, 1536) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert name(1, 1024, 4352, 1536) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    # dW whose 128 x 128 grid fills under 70% of its rounds: dY in registers
    assert name(2, 1024, 3072, 3072) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 1024, 4096, 4096) == "128x128x32_w2x2_sp4_pf3_il_dA"
    # dW whose 128 x 192 grid spans more than one round: dY in registers; one
    # whole round of 128 x 192 stays
    assert name(2, 1024, 2304, 3072) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 4096, 4608, 1792) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 1024, 2048, 3072) == "128x192x32_w2x2_sp8_pf4_il"
    assert name(2, 512, 768, 16384) == "128x128x32_w2x2_sp4_pf3_il_dA"
    assert name(1, 32768, 16, 768) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert name(2, 1024, 768, 768) == "48x48x64_k4_sp4_pf3_dAW"
    assert name(2, 1024, 512, 512) == "48x48x64_k4_sp4_pf2_ks2_dAW"
    assert name(2, 2048, 512, 512) == "48x48x64_k4_sp4_pf2_ks4_dAW"
    assert name(2, 8192, 384, 768) == "48x48x64_k4_sp4_pf2_ks4_dAW"
    assert name(2, 8192, 512, 512, ws=0) == "48x48x64_k4_sp4_pf3_dAW"
    assert name(2, 2048, 1024, 1024) == "48x48x64_k4_sp4_pf3_dAW"
    assert name(2, 4096, 768, 1536) == "48x48x64_k4_sp4_pf3_dAW"
    assert name(2, 8192, 1024, 1024) == "48x48x64_k4_sp4_pf2_ks2_dAW"
    # dW whose 32 x 96 grid fills whole rounds: dY into registers, whatever
    # the contraction
    assert name(2, 8192, 768, 3072) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 8192, 1024, 4096) == "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert name(2, 512, 1024, 1024) == "64x48x64_w2x1_k2_sp4_pf3_il_dA"
    assert lib.gemm_bwd_config_name(lib.gemm_bwd_select_config(2, 8192, 3072, 768, 1, 1)).decode() == \
        "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"
    assert lib.gemm_bwd_config_name(lib.gemm_bwd_select_config(2, 512, 3072, 768, 1, 1)).decode() == \
        "32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"


def test_loss_exports_and_validation(lib):
    """include/loss.h: every declared function is exported, and bad arguments
    are rejected synchronously (fake host pointers, nothing launched)."""
    with open(os.path.join(ROOT, "include", "loss.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(loss_[a-z_]+)\s*\(", text)))
    assert names == ["loss_cross_entropy", "loss_sum_losses"]
    for n in names:
        assert hasattr(lib, n)
    NULL, SHAPE, ALIGN = _status("GEMM_ERR_NULL"), _status("GEMM_ERR_SHAPE"), _status("GEMM_ERR_ALIGN")
    DTYPE, ALIAS = _status("GEMM_ERR_DTYPE"), _status("GEMM_ERR_ALIAS")
    ce = lambda l=X, t=W, o=Y, S=8, V=64, a=0.0, b=0.0, n=1.0: lib.loss_cross_entropy(l, t, o, S, V, a, b, n, None)
    assert ce(S=-1) == SHAPE and ce(V=-1) == SHAPE and ce(V=1 << 29) == SHAPE
    assert ce(l=None) == NULL and ce(t=None) == NULL and ce(o=None) == NULL
    assert ce(l=X + 2) == ALIGN and ce(t=W + 1) == ALIGN and ce(o=Y + 3) == ALIGN
    assert ce(a=-0.1) == DTYPE and ce(a=1.5) == DTYPE and ce(b=-1.0) == DTYPE
    assert ce(b=float("inf")) == DTYPE and ce(n=float("nan")) == DTYPE
    assert ce(o=X + 64) == ALIAS and ce(o=W) == ALIAS
    assert ce(S=0) == 0 and ce(S=0, l=None, t=None, o=None) == 0
    sl = lambda x=X, o=Y, S=8: lib.loss_sum_losses(x, o, S, None)
    assert sl(S=-1) == SHAPE and sl(o=None) == NULL and sl(x=None) == NULL and sl(x=X + 2) == ALIGN
    assert sl(o=X + 4) == ALIAS


def test_activation_exports_and_validation(lib):
    with open(os.path.join(ROOT, "include", "activation.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(act_[a-z_]+)\s*\(", text)))
    assert names == ["act_ffn_gelu_backward", "act_ffn_swiglu_backward", "act_gelu_inplace"]
    for n in names:
        assert hasattr(lib, n)
    NULL, SHAPE, ALIGN, ALIAS = (_status(s) for s in ("GEMM_ERR_NULL", "GEMM_ERR_SHAPE", "GEMM_ERR_ALIGN",
                                                       "GEMM_ERR_ALIAS"))
    sw = lambda g=X, x=W, u=U, dg=Y, du=R, n=64: lib.act_ffn_swiglu_backward(g, x, u, dg, du, n, None)
    assert sw(n=-1) == SHAPE and sw(n=0) == 0 and sw(g=None) == NULL and sw(du=None) == NULL
    assert sw(x=W + 2) == ALIGN and sw(dg=R) == ALIAS and sw(dg=X + 16) == ALIAS and sw(du=Y + 128) == ALIAS
    gb = lambda g=X, x=W, d=Y, n=64: lib.act_ffn_gelu_backward(g, x, d, n, None)
    assert gb(n=-1) == SHAPE and gb(x=None) == NULL and gb(d=Y + 1) == ALIGN and gb(d=W + 4) == ALIAS
    gi = lambda x=X, p=Y, n=64: lib.act_gelu_inplace(x, p, n, None)
    assert gi(x=None) == NULL and gi(p=X) == ALIAS and gi(p=X + 8) == ALIAS and gi(n=0) == 0
