"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two test programs under tests/sanitize/: the oracle built by g++ with both
sanitizers (brute-force products in every variant, row subsets, binary16
weights, the decoder over every pattern, row/column sums, argument checks),
and the library's host code built by hipcc with the sanitizers on the host
side only (every entry point's validation, extreme and overflowing shapes,
workspace errors, the tile-choice and workspace-size queries over a sweep of
shapes; nothing is launched).  The builds are cached under _build/sanitize,
keyed by the sources and flags, so only a change rebuilds them."""
import hashlib
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
PKG = os.path.join(ROOT, "tiled_dense_gemm_matmul_amd")
LIB_SRCS = [os.path.join(PKG, "csrc", f) for f in ("gemm_fwd.hip", "loss.hip", "activation.hip")]
HEADERS = [os.path.join(ROOT, "include", f) for f in ("gemm_fwd.h", "loss.h", "activation.h")]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _cached_build(name, cmd, inputs):
    h = hashlib.sha256(" ".join(cmd).encode())
    for path in inputs:
        with open(path, "rb") as f:
            h.update(f.read())
    exe = os.path.join(OUT, f"{name}-{h.hexdigest()[:16]}")
    if not os.path.exists(exe):
        os.makedirs(OUT, exist_ok=True)
        subprocess.run(cmd + ["-o", exe + ".tmp"], check=True, capture_output=True, text=True)
        os.replace(exe + ".tmp", exe)
    return exe


def test_oracle_under_sanitizers():
    src = [os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(ROOT, "tests", "sanitize", "oracle_checks.cpp")]
    cmd = ["g++", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fopenmp",
           "-ffp-contract=off", "-std=c++17", *src]
    exe = _cached_build("oracle_checks", cmd, src)
    r = subprocess.run([exe], env=ENV, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle checks ok" in r.stdout


def test_library_host_code_under_sanitizers():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    prog = os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp")
    # instrumentation on the host side only: each -fsanitize= right after -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *LIB_SRCS, prog]
    exe = _cached_build("host_checks", cmd, LIB_SRCS + HEADERS + [prog])
    r = subprocess.run([exe], env=ENV, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout
