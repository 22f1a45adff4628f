"""Build libgemmfwd.so (HIP, gfx950) in-tree with hipcc.

The packed-fp32 target feature is switched off for every HIP translation unit:
the kernels' fp32 arithmetic is scalar VALU plus MFMA.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_fwd.hip")
LOSS_SRC = os.path.join(PKG, "csrc", "loss.hip")
ACT_SRC = os.path.join(PKG, "csrc", "activation.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemmfwd.so")
SYNC_LIB = os.path.join(PKG, "libgemmfwd_sync.so")
PROBE_SRC = os.path.join(PKG, "csrc", "mfma_probe.hip")
PROBE_LIB = os.path.join(PKG, "libmfmaprobe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(srcs, lib: str, verbose: bool, defines=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_library(verbose: bool = False) -> str:
    """The library: the GEMM family (forward and backward), the fused loss and
    the FFN activation kernels."""
    return _hipcc([SRC, LOSS_SRC, ACT_SRC], LIB, verbose)


def build_sync_check_library(verbose: bool = False) -> str:
    """The verification build of the same sources (GEMM_SYNC_CHECK: full
    waits before every barrier, fences around the split-K exchange), which
    the race-check tests compare bit for bit with the shipping library."""
    return _hipcc([SRC, LOSS_SRC, ACT_SRC], SYNC_LIB, verbose, defines=("GEMM_SYNC_CHECK",))


def build_probe(verbose: bool = False) -> str:
    """The MFMA ceiling probe used by bench.py --mfma-ceiling."""
    return _hipcc([PROBE_SRC], PROBE_LIB, verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_sync_check_library(verbose=True))
    print(build_probe(verbose=True))
