"""Throughput of the forward linear-layer GEMM family on one MI355X.

One step is one forward pass of the fused GEMM family over a 512-token batch
with the model shape of the pages (d_model 768, d_ff 3072, vocabulary 16384):

  qkvo_residual   matmul_residual            512 x 768  x 768    fp32 W, +R
  qkvo            matmul                     512 x 768  x 768    fp32 W
  ffn_down        matmul_residual_swiglu_a   512 x 3072 x 768    fp32 W, +R
  ffn_gate_up     matmul_w16                 512 x 768  x 3072   f16 W
  lm_head         matmul_w16                 512 x 768  x 16384  f16 W

so every stage of the path runs in each step (plain and SwiGLU A staging,
fp32 and binary16 B staging, with and without the residual epilogue).
Inputs are the seeded synthetic arrays of the parity tests, resident in HBM
before the timed region.  The value is TFLOP/s = 2*M*N*K summed over the step,
divided by the wall time per step.  The roofline object describes the
dominant kernel (lm_head) against the fp32 matrix-core peak of MI355X, with
its average duration taken from HIP events that the launch itself records at
the kernel's start and end (gemm_opts.start_event / stop_event of the _ex
entry points) for each of its launches in the timed region.  The events are
the library's timing events (gemm_timing_event_create): a default HIP timing
event writes back and invalidates the caches at system scope when it is
recorded, which lengthens the timed kernel by about 2 us and delays the next
launch by about 5 us per step; these record the same start and end times
without it.  Every product
goes through the _ex entry points with a workspace sized by
gemm_fwd_workspace_bytes (only the SwiGLU down-projection splits K and uses
it), allocated before the timed region.  The per-kernel breakdown comes from a separate pass after the
timed region with such events on every launch.

The CPU baseline is the fp64 oracle, timed on whole steps of the same five
products (repeated for at least --cpu-seconds), on this host's cores.

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
this script (FETCH_SIZE, then WRITE_SIZE) and two of its --copy-calibration
mode (a plain device copy of a known size), turned into bytes per launch by
--traffic-from (for every kernel of the step) and kept in
profiles/lm_head_traffic.json together with the hash of the kernel's device
code (and of the lm_head tile's table entry) they were taken on; the bench
line reports them only while that hash still matches and the library still
picks that tile.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3   # 256 CU x 256 flop/clk/CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "TFLOP/s of fused forward GEMMs (seq 512, d768/3072/16384); % FP32 MFMA peak"
KERNEL_SRC = os.path.join(ROOT, "tiled_dense_gemm_matmul_amd", "csrc", "gemm_fwd.hip")
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "lm_head_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="seconds of untimed steps run before the counted warm-up, so that the engine "
                         "clock has ramped after the host-side input generation (reported as prewarm_s)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the step: time every workload configuration alone (warm median/min/p90, "
                         "cold-cache HBM GB/s for the N=768 shapes, torch.matmul fp32 as context) and print "
                         "a markdown table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of COPY_BYTES (for counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the step: time the backward products (matmul_t, matmul_at, _acc, "
                         "_swiglu_a) at the seq-512 model's shapes and print a markdown table")
    ap.add_argument("--loss", action="store_true",
                    help="instead of the step: time the fused loss (cross_entropy in place, sum_losses) on the "
                         "seq-512 logits and on the 16 x 512-token batch's, warm and cold, against HBM bandwidth")
    ap.add_argument("--activation", action="store_true",
                    help="instead of the step: time the FFN activation kernels (ffn_swiglu_backward, "
                         "ffn_gelu_backward, gelu_inplace) at the seq-512 and 8192-token hidden sizes")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the step: run the MFMA ceiling probe (independent fp32 MFMAs only) at 4, 8 "
                         "and 16 waves per CU and print the sustained TFLOP/s and engine clock")
    ap.add_argument("--shards", action="store_true",
                    help="instead of the step: time each product at the per-GPU shape of its natural sharding "
                         "over 2, 4 and 8 GPUs (lm_head and gate/up by columns, the SwiGLU down-projection by "
                         "its contraction), one GPU standing in for one shard")
    ap.add_argument("--counter-workloads", action="store_true",
                    help="instead of the step: launch cfg1 and the 16 x 512-token products (M = 8192 and 8191) "
                         "in turn a few times, for rocprofv3 counter runs")
    ap.add_argument("--counters-from", metavar="DIR",
                    help="turn the rocprofv3 counter runs under DIR (step/p1, step/p2, workloads/p1, workloads/p2) "
                         "into the counter summaries under profiles/ and exit")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="with or without --counters-from: turn the FETCH_SIZE / WRITE_SIZE runs under DIR "
                         "(step/fetch, step/write, workloads/..., copy_fetch, copy_write) into the traffic "
                         "summaries under profiles/ and " + os.path.relpath(TRAFFIC_FILE, ROOT) + ", and exit")
    ap.add_argument("--trace-from", metavar="DIR",
                    help="turn a rocprofv3 --kernel-trace run of the step (DIR/trace) and the bench line it "
                         "printed (DIR/bench.log) into profiles/seq512_step_kernel_trace.md and exit")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration():
    import torch
    x = torch.ones(COPY_BYTES // 4, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes 5 times", flush=True)


BACKWARD = [
    # label, op, M, K, N (forward names: M tokens, K inputs, N outputs)
    ("qkvo dX", "matmul_t", 512, 768, 768),
    ("ffn_down dH", "matmul_t", 512, 3072, 768),
    ("ffn_gate_up dX", "matmul_t_acc", 512, 768, 3072),
    ("lm_head dX", "matmul_t", 512, 768, 16384),
    ("qkvo dW", "matmul_at", 512, 768, 768),
    ("ffn_gate_up dW", "matmul_at_acc", 512, 768, 3072),
    ("ffn_down dW (SwiGLU recomputed)", "matmul_at_swiglu_a", 512, 3072, 768),
    ("lm_head dW", "matmul_at", 512, 768, 16384),
    # the 16 x 512-token batch
    ("qkvo dX, 8192 tokens", "matmul_t", 8192, 768, 768),
    ("ffn_down dH, 8192 tokens", "matmul_t", 8192, 3072, 768),
    ("ffn_gate_up dX, 8192 tokens", "matmul_t_acc", 8192, 768, 3072),
    ("qkvo dW, 8192 tokens", "matmul_at", 8192, 768, 768),
    ("ffn_gate_up dW, 8192 tokens", "matmul_at_acc", 8192, 768, 3072),
    ("ffn_down dW (SwiGLU recomputed), 8192 tokens", "matmul_at_swiglu_a", 8192, 3072, 768),
]


def time_backward():
    """The backward products at the seq-512 model's shapes, each on its own:
    batches of back-to-back launches queued behind busy_blocker(), between two
    timing-event markers (so the figure includes the launch gaps), after at
    least 0.2 s of warm-up; torch.matmul in fp32 on the same plain product as
    context."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    dev = torch.device("cuda:0")
    rows = []
    lines = ["| product | kernel | M×K×N (forward names) | output | µs per launch | TFLOP/s | % of 157.3 | "
             "torch.matmul fp32 µs |", "|---|---|---|---|---|---|---|---|"]
    for label, op, M, K, N in BACKWARD:
        c = inputs.backward_case(M + K + N, M, K, N, swiglu="swiglu" in op, acc="acc" in op)
        t = {k: torch.from_numpy(v).to(dev) for k, v in c.items()}
        acc = "acc" in op
        if op.startswith("matmul_t"):
            out = t["dX0"].clone() if acc else torch.empty((M, K), device=dev)
            run = lambda: binding.matmul_t(t["dY"], t["W"], out=out, acc=acc)
            ref = lambda: torch.matmul(t["dY"], t["W"].t())
            kcfg = binding.bwd_kernel_config("matmul_t", M, K, N)
        else:
            out = t["dW0"].clone() if acc else torch.empty((K, N), device=dev)
            if "swiglu" in op:
                run = lambda: binding.matmul_at_swiglu_a(t["G"], t["U"], t["dY"], out=out, acc=acc)
                ref = lambda: torch.matmul((torch.nn.functional.silu(t["G"]) * t["U"]).t(), t["dY"])
            else:
                run = lambda: binding.matmul_at(t["X"], t["dY"], out=out, acc=acc)
                ref = lambda: torch.matmul(t["X"].t(), t["dY"])
            kcfg = binding.bwd_kernel_config("matmul_at", M, K, N, swiglu="swiglu" in op)

        batch = batch_time
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            batch(run, 10)
        us = float(np.median([batch(run, 50) for _ in range(5)]))
        for _ in range(3):
            ref()
        tus = float(np.median([batch(ref, 20) for _ in range(3)]))
        flops = 2 * M * K * N
        tf = flops / us / 1e6
        shape_out = f"{M}×{K}" if op.startswith("matmul_t") else f"{K}×{N}"
        row = {"product": label, "op": op, "M": M, "K": K, "N": N, "tile": kcfg, "us": round(us, 2),
               "tflops": round(tf, 2), "frac_fp32_mfma_peak": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
               "torch_matmul_fp32_us": round(tus, 2)}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        lines.append(f"| {label} | {op} [{kcfg}] | {M}×{K}×{N} | {shape_out} | {us:.2f} | {tf:.1f} | "
                     f"{100 * tf / PEAK_FP32_MFMA_TFLOPS:.1f} | {tus:.2f} |")
    # the FFN down-projection's input gradient followed by the SwiGLU backward:
    # two launches through HBM (dH written and read back) against the fused one
    M, K, N = 512, 3072, 768
    c = inputs.backward_case(7, M, K, N)
    rng = np.random.default_rng(8)
    t = {k: torch.from_numpy(v).to(dev) for k, v in c.items()}
    G = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32) * np.float32(3.0)).to(dev)
    U = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(dev)
    dH, dG, dU = (torch.empty((M, K), device=dev) for _ in range(3))

    def two():
        binding.matmul_t(t["dY"], t["W"], out=dH)
        binding.ffn_swiglu_backward(dH, G, U, grad_gate=dG, grad_up=dU)

    def fused():
        binding.matmul_t_swiglu_backward(t["dY"], t["W"], G, U, grad_gate=dG, grad_up=dU)

    res = {}
    for name, fn in (("separate", two), ("fused", fused)):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            fn()
            torch.cuda.synchronize()
        res[name] = batch_time(fn, 50)
    print(json.dumps({"ffn_down_dH_and_swiglu_backward_us": {k: round(v, 2) for k, v in res.items()}}),
          file=sys.stderr, flush=True)
    lines += ["", f"FFN down-projection input gradient + SwiGLU backward ({M}×{K}×{N}): matmul_t then "
                  f"ffn_swiglu_backward {res['separate']:.2f} µs; fused (gemm_matmul_t_swiglu_bwd, dH never "
                  f"stored) {res['fused']:.2f} µs."]
    print("\n".join(lines))
    return rows


def time_loss():
    """cross_entropy over the lm_head logits, each launch between its own
    pair of timing-event markers (median of the launches, all queued behind
    busy_blocker()), warm (logits of the seq-512 step fit
    the 256 MB Infinity Cache) and cold (a 512 MiB buffer written between
    launches).  The kernel rewrites the logits in place, so later launches
    see gradients rather than logits; the work does not depend on the values.
    Algorithmic bytes: the logits read once and written once, plus targets
    and losses."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    flush = torch.empty(128 << 20, device=dev)
    lines = ["| logits S×V | path | warm median µs | warm GB/s | cold median µs | cold GB/s | % of 8 TB/s (cold) | "
             "sum_losses µs |", "|---|---|---|---|---|---|---|---|"]
    rows = []
    for S, V in ((512, 16384), (8192, 50304)):
        c = inputs.loss_case(S + V, S, V, ignore_every=97)
        logits = torch.from_numpy(c["logits"]).to(dev)
        tg = torch.from_numpy(c["targets"].astype(np.int32)).to(dev)
        losses = torch.empty(S, device=dev)
        inv = 1.0 / int((c["targets"] < V).sum())
        lib = binding.load_library()
        # the C entry point directly, so that the events see only the kernel
        run = lambda: lib.loss_cross_entropy(logits.data_ptr(), tg.data_ptr(), losses.data_ptr(), S, V, 0.1, 1e-4,
                                             inv, st.cuda_stream)

        def sample(n, cold):
            return float(np.median(marker_times(run, n, (lambda: flush.fill_(1.0)) if cold else None)))

        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            run()
            torch.cuda.synchronize()
        n = 50 if S * V < 1e8 else 10
        warm, cold = sample(n, False), sample(n, True)
        total = torch.empty(1, device=dev)
        sl_us = batch_time(lambda: lib.loss_sum_losses(losses.data_ptr(), total.data_ptr(), S, st.cuda_stream), 20)
        nbytes = 2 * S * V * 4 + 2 * S * 4
        # the library's launch shape for rows of V logits (16-byte accesses)
        shape = next(((nt, cap) for nt, cap, lim in ((256, 16, 4096), (512, 16, 8192), (512, 32, 16384),
                                                      (1024, 32, 32768), (1024, 64, 65536)) if V <= lim), None)
        path = f"registers, {shape[0]} threads x {shape[1]} logits/row" if shape and V % 4 == 0 else \
            ("registers, 256 threads x 64 logits/row" if V <= 16384 else "streaming")
        row = {"S": S, "V": V, "warm_us": round(warm, 2), "warm_GBps": round(nbytes / warm / 1e3, 1),
               "cold_us": round(cold, 2), "cold_GBps": round(nbytes / cold / 1e3, 1),
               "frac_hbm_peak_cold": round(nbytes / cold / 1e3 / PEAK_HBM_GBS, 4), "sum_losses_us": round(sl_us, 2)}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        lines.append(f"| {S}×{V} | {path} | {warm:.2f} | {nbytes / warm / 1e3:.0f} | {cold:.2f} | "
                     f"{nbytes / cold / 1e3:.0f} | {100 * nbytes / cold / 1e3 / PEAK_HBM_GBS:.1f} | {sl_us:.2f} |")
        del logits
        torch.cuda.empty_cache()
    print("\n".join(lines))
    return rows


def time_activation():
    """The FFN activation kernels on their own, each launch between its own
    pair of timing-event markers around the C entry point (median, all queued
    behind busy_blocker()), warm and cold (a 512 MiB
    buffer written between launches).  Algorithmic bytes per element:
    ffn_swiglu_backward reads three arrays and writes two (20 B),
    ffn_gelu_backward reads two and writes one (12 B), gelu_inplace reads
    and writes one and keeps a copy of the input (12 B)."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    lib = binding.load_library()
    flush = torch.empty(128 << 20, device=dev)
    lines = ["| kernel | elements | bytes/elem | warm µs | warm GB/s | cold µs | cold GB/s | % of 8 TB/s (cold) |",
             "|---|---|---|---|---|---|---|---|"]
    rows = []
    for n in (512 * 3072, 8192 * 3072):
        c = inputs.activation_case(n % 1000 + 1, n)
        g, x, u = (torch.from_numpy(c[k]).to(dev) for k in ("g", "gate", "up"))
        o1, o2 = torch.empty_like(g), torch.empty_like(g)
        kernels = [
            ("ffn_swiglu_backward", 20, lambda: lib.act_ffn_swiglu_backward(
                g.data_ptr(), x.data_ptr(), u.data_ptr(), o1.data_ptr(), o2.data_ptr(), n, st.cuda_stream)),
            ("ffn_gelu_backward", 12, lambda: lib.act_ffn_gelu_backward(
                g.data_ptr(), x.data_ptr(), o1.data_ptr(), n, st.cuda_stream)),
            ("gelu_inplace (keeping the input)", 12, lambda: lib.act_gelu_inplace(
                o2.data_ptr(), o1.data_ptr(), n, st.cuda_stream)),
        ]
        for name, bpe, run in kernels:
            def sample(k, cold):
                return float(np.median(marker_times(run, k, (lambda: flush.fill_(1.0)) if cold else None)))
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.2:
                run()
                torch.cuda.synchronize()
            warm, cold = sample(50, False), sample(50, True)
            nbytes = bpe * n
            row = {"kernel": name, "n": n, "warm_us": round(warm, 2), "warm_GBps": round(nbytes / warm / 1e3, 1),
                   "cold_us": round(cold, 2), "cold_GBps": round(nbytes / cold / 1e3, 1),
                   "frac_hbm_peak_cold": round(nbytes / cold / 1e3 / PEAK_HBM_GBS, 4)}
            rows.append(row)
            print(json.dumps(row), file=sys.stderr, flush=True)
            lines.append(f"| {name} | {n} | {bpe} | {warm:.2f} | {nbytes / warm / 1e3:.0f} | {cold:.2f} | "
                         f"{nbytes / cold / 1e3:.0f} | {100 * nbytes / cold / 1e3 / PEAK_HBM_GBS:.1f} |")
    print("\n".join(lines))
    return rows


def mfma_ceiling():
    """What the fp32 matrix cores sustain with nothing but independent MFMAs
    in flight: the ceiling that the roofline's published peak stands for."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "tiled_dense_gemm_matmul_amd", "libmfmaprobe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.mfma_probe_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mfma_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.mfma_probe_flops.restype = ctypes.c_longlong
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    iters, reps = 8192, 10
    out = []
    for waves_per_cu in (4, 8, 16):
        blocks = 256 * waves_per_cu // 4
        sink = torch.empty(blocks * 256, device=dev)
        clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)

        def launch():
            rc = lib.mfma_probe_launch(sink.data_ptr(), clocks.data_ptr(), blocks, iters, st.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"mfma_probe_launch returned {rc}")

        # clocks ramp after host-side work: warm up for at least 0.3 s
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            launch()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            launch()
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        c = clocks.view(blocks, 2).cpu().double()
        mhz = float(c[:, 0].sum() / c[:, 1].sum() * 100.0)
        tflops = lib.mfma_probe_flops(blocks, iters) / (ms * 1e-3) / 1e12
        out.append({"waves_per_cu": waves_per_cu, "ms": round(ms, 4), "tflops": round(tflops, 1),
                    "frac_of_peak": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4), "clock_mhz": round(mhz)})
        print(json.dumps(out[-1]), flush=True)
    return out


COUNTER_PASSES = {
    "p1": "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
          "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_MFMA SQ_INSTS_VALU GRBM_GUI_ACTIVE",
    "p2": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS SQ_VALU_MFMA_COEXEC_CYCLES "
          "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
}
STEP_LABELS = ["qkvo_residual", "qkvo", "ffn_down", "ffn_gate_up", "lm_head"]   # launch order in a step

# The kernels of each counter set in launch order: label, M, K, N, SwiGLU,
# f16 W, residual.  "step" is the seq-512 step (bench.py --steps 5 --warmup 2
# --prewarm-s 0 --no-cpu); "workloads" the other workload configurations
# (bench.py --counter-workloads), launched WORKLOAD_REPS times in turn.
COUNTER_SETS = {
    "step": {
        "title": "the seq-512 forward step (bench.py)",
        "cmd": "python3 $R/bench.py --steps 5 --warmup 2 --prewarm-s 0 --no-cpu",
        "kernels": [("qkvo_residual", 512, 768, 768, False, False, True),
                    ("qkvo", 512, 768, 768, False, False, False),
                    ("ffn_down", 512, 3072, 768, True, False, True),
                    ("ffn_gate_up", 512, 768, 3072, False, True, False),
                    ("lm_head", 512, 768, 16384, False, True, False)],
        "counters_md": "seq512_counters.md", "traffic_md": "seq512_traffic.md",
    },
    "workloads": {
        "title": "the 128-token and 16 x 512-token workloads (bench.py --counter-workloads)",
        "cmd": "python3 $R/bench.py --counter-workloads",
        "kernels": [("cfg1 matmul", 128, 768, 768, False, False, False),
                    ("cfg5a SwiGLU+R, M=8192", 8192, 3072, 768, True, True, True),
                    ("cfg5a SwiGLU+R, M=8191", 8191, 3072, 768, True, True, True),
                    ("cfg5b lm_head, M=8192", 8192, 768, 50304, False, True, False),
                    ("cfg5b lm_head, M=8191", 8191, 768, 50304, False, True, False)],
        "counters_md": "workload_counters.md", "traffic_md": "workload_traffic.md",
    },
}
WORKLOADS = [
    # the "workloads" counter set: generator, variant keys, M rows used
    ("cfg1", ("X", "W", None), None),
    ("cfg5", ("G", "U", "W_down", "R"), None),
    ("cfg5", ("G", "U", "W_down", "R"), 8191),
    ("cfg5", ("X", "W_lm", None), None),
    ("cfg5", ("X", "W_lm", None), 8191),
]
WORKLOAD_REPS = 3


def alg_bytes(M, K, N, swiglu, w16, resid):
    """Algorithmic HBM bytes of one launch: A (G and U with SwiGLU) and W
    read once, R read once, Y written once."""
    return M * K * (8 if swiglu else 4) + K * N * (2 if w16 else 4) + M * N * 4 * (2 if resid else 1)


def counter_workloads():
    """The "workloads" counter set: each configuration in the library's
    choice (with its workspace), all launched in turn WORKLOAD_REPS times."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    lib = binding.load_library()
    dev = torch.device("cuda:0")
    sp = torch.cuda.current_stream(dev).cuda_stream
    gens, launches = {}, []
    for (gen, keys, rows), spec in zip(WORKLOADS, COUNTER_SETS["workloads"]["kernels"]):
        if gen not in gens:
            gens[gen] = getattr(inputs, gen)()
        c = gens[gen]

        def d(key, r=None):
            a = c[key]
            return torch.from_numpy(np.ascontiguousarray(a if r is None else a[:r])).to(dev)
        swiglu = len(keys) == 4
        if swiglu:
            ts = [d(keys[0], rows), d(keys[1], rows)]
            W, rkey = d(keys[2]), keys[3]
        else:
            ts = [d(keys[0], rows)]
            W, rkey = d(keys[1]), keys[2]
        R = d(rkey, rows) if rkey else None
        M, K = ts[0].shape
        N = W.shape[1]
        w16 = W.dtype == torch.float16
        assert (M, K, N, swiglu, w16, R is not None) == spec[1:], (spec, M, K, N)
        Y = torch.empty((M, N), device=dev)
        wsb = lib.gemm_fwd_workspace_bytes(M, K, N, int(swiglu), int(w16), -1)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
        o = binding.opts(-1, ws.data_ptr() if wsb else None, wsb)
        if swiglu:
            a = (ts[0].data_ptr(), ts[1].data_ptr(), W.data_ptr(), R.data_ptr(), Y.data_ptr(), M, K, N, int(w16))
            launches.append((spec[0], lib.gemm_fwd_swiglu_ex, a, o, (ts, W, R, Y, ws)))
        else:
            a = (ts[0].data_ptr(), W.data_ptr(), None if R is None else R.data_ptr(), Y.data_ptr(), M, K, N,
                 binding.GEMM_FLAG_W_F16 if w16 else 0)
            launches.append((spec[0], lib.gemm_fwd_ex, a, o, (ts, W, R, Y, ws)))
    torch.cuda.synchronize()
    for rep in range(WORKLOAD_REPS):
        for label, fn, a, o, _ in launches:
            st = fn(*a, o, sp)
            if st != 0:
                raise RuntimeError(f"{label}: {binding.status_string(st)}")
        torch.cuda.synchronize()
        print(f"counter workloads: round {rep + 1} of {WORKLOAD_REPS} done", flush=True)


def _gemm_rows(run_dir, what="counter_collection"):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", f"*{what}.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no {what}.csv under {run_dir}")
    with open(files[0]) as f:
        return [r for r in csv.DictReader(f) if "gemm_fwd_kernel" in r["Kernel_Name"]]


def _by_kernel(rows, labels):
    """Counter rows grouped by the kernel of the set that each dispatch is
    (dispatch order modulo the set's launches)."""
    import collections
    order = {d: i for i, d in enumerate(sorted({int(r["Dispatch_Id"]) for r in rows}))}
    if len(order) % len(labels):
        raise SystemExit(f"{len(order)} GEMM dispatches is not a whole number of rounds of {len(labels)}")
    out = collections.defaultdict(list)
    for r in rows:
        out[labels[order[int(r["Dispatch_Id"])] % len(labels)]].append(r)
    return out


def counters_table(base, set_name):
    """Per-kernel hardware counters of a counter set from its two
    rocprofv3 --pmc runs (base/<set>/p1, p2), as markdown."""
    import collections
    import statistics
    cs = COUNTER_SETS[set_name]
    labels = [k[0] for k in cs["kernels"]]
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    clocks = collections.defaultdict(list)
    for run in COUNTER_PASSES:
        for k, rows in _by_kernel(_gemm_rows(os.path.join(base, set_name, run)), labels).items():
            for r in rows:
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
                    durs[k].append(dur)
                    clocks[k].append(float(r["Counter_Value"]) / 8 / dur)
    simds = 1024
    lines = [
        f"# Hardware counters of {cs['title']}",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root on the GPU host and $OUT an output "
        "directory), one counter set per run:",
        "",
    ]
    for run, ctrs in COUNTER_PASSES.items():
        lines.append(f"    timeout -s KILL 120 rocprofv3 --pmc {ctrs} -f csv -d $OUT/counters/{set_name}/{run} -o pmc -- "
                     f"{cs['cmd']}")
    lines += [
        "    python3 bench.py --counters-from $OUT/counters      # writes this file",
        "",
        "Averages over every launch of each kernel in those runs.  Counter collection serialises launches and",
        "slows the kernels (the `µs under counters` column), so the busy fractions are lower than in an",
        "unprofiled run; the instruction counts are exact.",
        "",
        "- MFMA count / ideal = SQ_INSTS_MFMA / (2MNK / 2048), the flops of one v_mfma_f32_16x16x4_f32",
        "  (partial tiles are padded to whole 16 x 16 blocks, so a ragged M or N counts above 1).",
        "- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (32 per MFMA, summed over SIMDs) / (1024 SIMDs x 2400 MHz x duration).",
        "- clock = GRBM_GUI_ACTIVE / 8 XCDs / duration: the engine clock, shown for kernels of 50 us and more",
        "  (the counter also runs outside a short kernel's own start and end).",
        "- other VALU per MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA (the VALU count includes the MFMAs);",
        "  co-issue = SQ_VALU_MFMA_COEXEC_CYCLES, cycles in which a VALU instruction issued while the MFMA unit was busy.",
        "- LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS).",
        "",
        "| kernel | M×K×N | launches | µs under counters | clock MHz | MFMA count / ideal | MFMA busy | "
        "other VALU per MFMA | co-issue cycles | LDS instr per MFMA | LDS conflict | L2 hit |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for (k, M, K, N, *_rest) in cs["kernels"]:
        v = {c: statistics.mean(x) for c, x in vals[k].items()}
        d = statistics.median(durs[k])
        ideal = 2 * M * K * N / 2048
        lines.append(
            f"| {k} | {M}×{K}×{N} | {len(vals[k]['SQ_INSTS_MFMA'])} | {d:.1f} | "
            f"{f'{statistics.median(clocks[k]):.0f}' if d >= 50 else '—'} | "
            f"{v['SQ_INSTS_MFMA'] / ideal:.3f} | {100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * 2400 * d):.1f}% | "
            f"{(v['SQ_INSTS_VALU'] - v['SQ_INSTS_MFMA']) / v['SQ_INSTS_MFMA']:.2f} | "
            f"{v['SQ_VALU_MFMA_COEXEC_CYCLES']:.0f} | "
            f"{v['SQ_INSTS_LDS'] / v['SQ_INSTS_MFMA']:.3f} | "
            f"{100 * v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.1f}% | "
            f"{100 * v['TCC_HIT_sum'] / (v['TCC_HIT_sum'] + v['TCC_MISS_sum']):.1f}% |")
    return lines


def traffic_table(base, set_name):
    """HBM bytes per launch of each kernel of a counter set from its
    FETCH_SIZE and WRITE_SIZE runs (base/<set>/fetch, write), each scaled by
    what the same counter reads for a plain copy of COPY_BYTES (base/copy_fetch,
    copy_write), as markdown plus a dict per kernel."""
    import statistics
    cs = COUNTER_SETS[set_name]
    labels = [k[0] for k in cs["kernels"]]

    def copy_kib(run):
        import csv
        import glob
        f = glob.glob(os.path.join(base, run, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(base, run)}")
        with open(f[0]) as fh:
            vals = [float(r["Counter_Value"]) for r in csv.DictReader(fh) if "copy" in r["Kernel_Name"].lower()]
        return statistics.median(vals)

    f_scale = COPY_BYTES / (copy_kib("copy_fetch") * 1024)
    w_scale = COPY_BYTES / (copy_kib("copy_write") * 1024)
    fetch = {k: [float(r["Counter_Value"]) for r in rows]
             for k, rows in _by_kernel(_gemm_rows(os.path.join(base, set_name, "fetch")), labels).items()}
    write = {k: [float(r["Counter_Value"]) for r in rows]
             for k, rows in _by_kernel(_gemm_rows(os.path.join(base, set_name, "write")), labels).items()}
    lines = [
        f"# HBM traffic of {cs['title']}",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root on the GPU host and $OUT an output "
        "directory), one counter per run:",
        "",
        f"    timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/traffic/{set_name}/fetch -o pmc -- {cs['cmd']}",
        f"    timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/traffic/{set_name}/write -o pmc -- {cs['cmd']}",
        "    timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/traffic/copy_fetch -o pmc -- "
        "python3 $R/bench.py --copy-calibration",
        "    timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/traffic/copy_write -o pmc -- "
        "python3 $R/bench.py --copy-calibration",
        "    python3 bench.py --counters-from $OUT/counters --traffic-from $OUT/traffic      # writes this file",
        "",
        f"Calibration: a device copy of {COPY_BYTES >> 20} MiB reads FETCH_SIZE = {copy_kib('copy_fetch') / 1024:.0f} MiB "
        f"and WRITE_SIZE = {copy_kib('copy_write') / 1024:.0f} MiB per dispatch, so FETCH_SIZE is scaled by "
        f"{f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}.  Averages over every launch of each kernel; "
        f"hash of the kernels' device code and the lm_head tile's entry at measurement: {kernel_hash()}.",
        "",
        "Algorithmic bytes: A (G and U with SwiGLU) and W read once, R read once, Y written once.",
        "",
        "FETCH_SIZE and WRITE_SIZE count what the L2 caches read from and write to the memory side of the chip:",
        "each XCD's L2 fetches its own copy of whatever its tiles read, and reads that the 256 MB Infinity Cache",
        "serves count as well, so the fetched bytes are an upper bound of the HBM reads.",
        "",
        "| kernel | M×K×N | launches | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | fetched bytes | written bytes | "
        "algorithmic reads | algorithmic writes | fetched / alg. reads | written / alg. writes |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    per = {}
    for (k, M, K, N, swiglu, w16, resid) in cs["kernels"]:
        fk, wk = statistics.mean(fetch[k]), statistics.mean(write[k])
        fb, wb = fk * 1024 * f_scale, wk * 1024 * w_scale
        ar = alg_bytes(M, K, N, swiglu, w16, resid) - M * N * 4
        aw = M * N * 4
        per[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "fetch_size_kib_raw": round(fk, 1),
                  "write_size_kib_raw": round(wk, 1), "algorithmic_bytes": ar + aw,
                  "dispatches": {"fetch": len(fetch[k]), "write": len(write[k])},
                  "copy_scale": {"FETCH_SIZE": round(f_scale, 4), "WRITE_SIZE": round(w_scale, 4)}}
        lines.append(f"| {k} | {M}×{K}×{N} | {len(fetch[k])} | {fk:.1f} | {wk:.1f} | {fb:,.0f} | {wb:,.0f} | "
                     f"{ar:,} | {aw:,} | {fb / ar:.2f} | {wb / aw:.2f} |")
    return lines, per


def counters_from(counters_base, traffic_base=None, out_dir=PROFILES):
    """Write the counter (and, with traffic_base, the HBM traffic) summaries
    of every counter set found under the run directories into out_dir, and
    the lm_head's bytes per launch into the traffic file bench.py reads
    (lm_head_traffic.json there)."""
    for set_name, cs in COUNTER_SETS.items():
        if counters_base and os.path.isdir(os.path.join(counters_base, set_name)):
            lines = counters_table(counters_base, set_name)
            with open(os.path.join(out_dir, cs["counters_md"]), "w") as f:
                f.write("\n".join(lines) + "\n")
            print("\n".join(lines))
        if traffic_base and os.path.isdir(os.path.join(traffic_base, set_name)):
            lines, per = traffic_table(traffic_base, set_name)
            with open(os.path.join(out_dir, cs["traffic_md"]), "w") as f:
                f.write("\n".join(lines) + "\n")
            print("\n".join(lines))
            if set_name == "step":
                lm = per["lm_head"]
                out = {"kernel_sha256_16": kernel_hash(), "kernel": "lm_head (matmul_w16 512x768x16384)",
                       "tile": LM_HEAD_TILE, "bytes_per_launch": lm["fetch_bytes"] + lm["write_bytes"], **lm}
                with open(os.path.join(out_dir, os.path.basename(TRAFFIC_FILE)), "w") as f:
                    json.dump(out, f, indent=1)
                    f.write("\n")


def trace_from(base, out_dir=PROFILES):
    """profiles/seq512_step_kernel_trace.md from a rocprofv3 --kernel-trace
    --stats run of the step (base/trace) and the bench line that run printed
    (base/bench.log): every launch of each step kernel, and the launches of
    the timed region alone against the HIP-event figure the bench line
    reports for them."""
    import statistics
    with open(os.path.join(base, "bench.log")) as f:
        line = json.loads([l for l in f if l.startswith("{")][-1])
    rows = _gemm_rows(os.path.join(base, "trace"), "kernel_trace")
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    n = len(STEP_LABELS)
    steps, warm, pre = line["steps"], line["warmup"], line["prewarm_steps"]
    nb = min(steps, 50)
    if len(rows) != n * (pre + warm + steps + nb):
        raise SystemExit(f"{len(rows)} GEMM dispatches, expected {n} x ({pre} + {warm} + {steps} + {nb})")
    t0, t1 = n * (pre + warm), n * (pre + warm + steps)
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in rows]

    def pick(i, lo, hi):
        return [dur[j] for j in range(lo, hi) if j % n == i]

    flops = {k: 2 * M * K * N for (k, M, K, N, *_r) in COUNTER_SETS["step"]["kernels"]}
    cmd = ("rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace -o bench -- "
           f"python3 $R/bench.py --steps {steps} --warmup {warm} --no-cpu")
    lines = [
        "# Kernel trace of the seq-512 forward step (bench.py)",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root on the GPU host and $OUT an output "
        "directory):",
        "",
        "    python3 $R/bench.py > $OUT/bench_plain.log      # unprofiled, for comparison",
        f"    {cmd} > $OUT/bench.log",
        "    python3 bench.py --trace-from $OUT      # writes this file",
        "",
        f"Device-code hash {kernel_hash()}.  The run made {pre} time-based pre-warm steps, {warm} counted warm-up "
        f"steps, the {steps} timed steps and a pass of {nb} steps with events on every launch: "
        f"{len(rows)} GEMM launches in all.",
        "",
        "| kernel | timed-region launches | rocprof avg µs | min | max | % of 157.3 at avg | all launches | "
        f"rocprof avg µs (all) | event pass: rocprof avg µs | event pass: bench.py event avg µs |",
        "|---|---|---|---|---|---|---|---|---|---|",
    ]
    for i, k in enumerate(STEP_LABELS):
        t = pick(i, t0, t1)
        a = pick(i, 0, len(rows))
        e = pick(i, t1, len(rows))
        avg = statistics.mean(t)
        lines.append(f"| {k} | {len(t)} | {avg:.2f} | {min(t):.2f} | {max(t):.2f} | "
                     f"{100 * flops[k] / avg / 1e6 / PEAK_FP32_MFMA_TFLOPS:.1f} | {len(a)} | {statistics.mean(a):.2f} | "
                     f"{statistics.mean(e):.2f} | {line['kernels'][k]['avg_us']:.2f} |")
    lm = pick(STEP_LABELS.index("lm_head"), t0, t1)
    lines += [
        "",
        f"Same run, bench.py line: {line['ms_per_step'] * 1e3:.1f} us per step, {line['value']} TFLOP/s; its roofline "
        f"kernel lm_head averaged {line['roofline']['avg_us']} us by HIP events over the {steps} timed-region launches, "
        f"against {statistics.mean(lm):.2f} us by the trace over the same launches.  Under the profiler the events "
        "read a few microseconds long and the step runs slower.",
    ]
    plain = os.path.join(base, "bench_plain.log")
    if os.path.exists(plain):
        with open(plain) as f:
            pl = json.loads([l for l in f if l.startswith("{")][-1])
        lines += [
            "",
            f"The unprofiled run of the same command in the same session (bench_plain.log): "
            f"{pl['ms_per_step'] * 1e3:.1f} us per step, {pl['value']} TFLOP/s; lm_head averaged "
            f"{pl['roofline']['avg_us']} us by HIP events over its {pl['roofline']['launches']} timed-region launches "
            f"({100 * (pl['roofline']['avg_us'] / statistics.mean(lm) - 1):+.1f}% against the trace above), "
            f"{pl['roofline']['frac'] * 100:.1f}% of {PEAK_FP32_MFMA_TFLOPS} TFLOP/s.",
        ]
    out = os.path.join(out_dir, "seq512_step_kernel_trace.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


LM_HEAD_TILE = "128x128x32_w2x2_sp4_pf3_il_dA"


def kernel_hash(tile=LM_HEAD_TILE):
    """Hash of the device code of the kernel source (everything before its
    configuration table) and of `tile`'s entry in that table, with comments
    and blank space removed, so that only a change to that kernel's code
    makes stored counter results stale."""
    import re
    with open(KERNEL_SRC) as f:
        src = f.read()
    cut = src.index("// configuration table")
    entry = next(line for line in src[cut:].splitlines() if f'"{tile}"' in line)
    src = src[:cut] + "\n" + entry
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def workload():
    from tiled_dense_gemm_matmul_amd import inputs
    c2, c3, c4 = inputs.cfg2(), inputs.cfg3(), inputs.cfg4()
    return [
        ("qkvo_residual", {"X": c2["X"], "W": c2["W"], "R": c2["R"]}),
        ("qkvo", {"X": c2["X"], "W": c2["W"]}),
        ("ffn_down", {"G": c3["G"], "U": c3["U"], "W": c3["W"], "R": c3["R"]}),
        ("ffn_gate_up", {"X": c4["X"], "W": c4["W_gu"]}),
        ("lm_head", {"X": c4["X"], "W": c4["W_lm"]}),
    ]


def shape_of(case):
    A = case["G"] if "G" in case else case["X"]
    return A.shape[0], A.shape[1], case["W"].shape[1]


def cpu_model():
    """The host CPU's full model string: lscpu's "Model name" (with the vendor
    and family/model numbers), else /proc/cpuinfo's "model name"."""
    import subprocess
    fields = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    name = fields.get("Model name")
    if not name:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        name = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    name = name or "unknown"
    extra = [f"{k} {fields[k]}" for k in ("Vendor ID", "CPU family", "Model", "Socket(s)") if k in fields]
    return name + (f" ({', '.join(extra)})" if extra else "")


def cpu_baseline(cases, min_seconds):
    """The fp64 oracle on whole steps (every output row of the five
    products), repeated until at least min_seconds have passed."""
    import oracle
    oracle.build(force=False)
    # The GPU host gives each GPU job a share of 16 CPU threads (its
    # OMP_NUM_THREADS), whatever the affinity mask shows; use at most that.
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    threads = max(1, min(affinity, share, 16))
    step_flops = sum(2 * shape_of(c)[0] * shape_of(c)[1] * shape_of(c)[2] for _, c in cases)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for _, c in cases:
            A = c["G"] if "G" in c else c["X"]
            oracle.gemm(A, c["W"], R=c.get("R"), U=c.get("U"), threads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {
        "value": reps * step_flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "threads_used": threads,
        "affinity_cores": affinity,
        "logical_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{reps} whole steps (all rows of the 5 products, "
                  f"{reps * step_flops / 1e9:.1f} GFLOP of fp64) in {dt:.1f} s",
    }


CONFIGS = [
    # name, generator, variant keys, M rows used (None: all), cold GB/s reported
    ("cfg1 matmul", "cfg1", ("X", "W", None), None, True),
    ("cfg2 matmul_residual", "cfg2", ("X", "W", "R"), None, True),
    ("cfg2 matmul", "cfg2", ("X", "W", None), None, True),
    ("cfg3 matmul_residual_swiglu_a", "cfg3", ("G", "U", "W", "R"), None, True),
    ("cfg4 matmul_w16 lm_head", "cfg4", ("X", "W_lm", None), None, False),
    ("cfg4b matmul_w16 gate/up", "cfg4", ("X", "W_gu", None), None, False),
    ("cfg5a matmul_residual_swiglu_a_w16", "cfg5", ("G", "U", "W_down", "R"), None, True),
    ("cfg5a (M=8191)", "cfg5", ("G", "U", "W_down", "R"), 8191, True),
    ("cfg5b matmul_w16 lm_head", "cfg5", ("X", "W_lm", None), None, False),
    ("cfg5b (M=8191)", "cfg5", ("X", "W_lm", None), 8191, False),
]


_BLOCKER = []


def busy_blocker():
    """Queue a few milliseconds of real work (three 4096^3 fp32 products in
    torch) ahead of the launches to be timed, so that the host has enqueued
    them all before the first one runs and the GPU runs them back to back.
    A spin kernel would do the first part, but it leaves the GPU idle for
    those milliseconds, the engine clock drops, and the kernels after it run
    up to 12% slow until it has ramped again."""
    import torch
    if not _BLOCKER:
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn((4096, 4096), device="cuda", generator=g)
        _BLOCKER.extend([a, a.clone(), torch.empty_like(a)])
    a, b, c = _BLOCKER
    for _ in range(3):
        torch.mm(a, b, out=c)


def marker_times(run, n, between=None):
    """Durations (us) of n calls of `run` (a launch that records no events
    itself), each between two of the library's timing events recorded as
    markers, all queued behind busy_blocker() so that the GPU runs them back
    to back.  `between` enqueues work before each marker pair."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    st = torch.cuda.current_stream()
    evs = [(binding.TimingEvent(), binding.TimingEvent()) for _ in range(n)]
    busy_blocker()
    for a, b in evs:
        if between is not None:
            between()
        a.record(st)
        assert run() in (0, None)
        b.record(st)
    torch.cuda.synchronize()
    return np.array([a.elapsed_ms(b) * 1e3 for a, b in evs])


def batch_time(fn, n):
    """Microseconds per call of n calls of `fn` queued back to back behind
    busy_blocker(), between two timing-event markers (launch gaps included)."""
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    st = torch.cuda.current_stream()
    e0, e1 = binding.TimingEvent(), binding.TimingEvent()
    busy_blocker()
    e0.record(st)
    for _ in range(n):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) * 1e3 / n


def queued_launch_times(launch, n, between=None):
    """Durations (us) of n launches, each timed by the library's timing
    events, all queued behind busy_blocker() so that the GPU runs them back
    to back: a short kernel whose launch reaches an idle GPU (the host
    enqueueing slower than the kernel runs) measures about one dispatch
    latency (~4 us) longer.  `between` enqueues work before each launch
    (outside its events)."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding
    evs = [(binding.TimingEvent(), binding.TimingEvent()) for _ in range(n)]
    busy_blocker()
    for a, b in evs:
        if between is not None:
            between()
        assert launch((a.handle, b.handle)) == 0
    torch.cuda.synchronize()
    return np.array([a.elapsed_ms(b) * 1e3 for a, b in evs])


def time_configs():
    """Each workload configuration on its own, timed per launch by events
    that the launch records at the kernel's start and end.  Warm: back-to-
    back launches (inputs up to cfg 4 stay in the 256 MB Infinity Cache).
    Cold: a 512 MiB buffer is written between launches, outside the kernel's
    interval, so its inputs come from HBM.  torch.matmul in fp32 on the
    same (plain) product is reported as context only."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    lib = binding.load_library()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    sp = st.cuda_stream
    flush = torch.empty(128 << 20, device=dev)
    gens = {}

    def d(a, rows=None):
        a = np.ascontiguousarray(a if rows is None else a[:rows])
        return torch.from_numpy(a).to(dev)

    rows_out = []
    for name, gen, keys, rows, cold in CONFIGS:
        if gen not in gens:
            gens = {gen: getattr(inputs, gen)()}
        c = gens[gen]
        swiglu = len(keys) == 4
        if swiglu:
            G, U, W, R = d(c[keys[0]], rows), d(c[keys[1]], rows), d(c[keys[2]]), d(c[keys[3]], rows)
            M, K = G.shape
        else:
            X, W = d(c[keys[0]], rows), d(c[keys[1]])
            R = d(c[keys[2]], rows) if keys[2] else None
            M, K = X.shape
        N = W.shape[1]
        w16 = W.dtype == torch.float16
        Y = torch.empty((M, N), device=dev)
        wsb = lib.gemm_fwd_workspace_bytes(M, K, N, int(swiglu), int(w16), -1)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)

        def launch(ev=(None, None)):
            o = binding.opts(-1, ws.data_ptr() if wsb else None, wsb, *ev)
            if swiglu:
                return lib.gemm_fwd_swiglu_ex(G.data_ptr(), U.data_ptr(), W.data_ptr(), R.data_ptr(),
                                              Y.data_ptr(), M, K, N, int(w16), o, sp)
            return lib.gemm_fwd_ex(X.data_ptr(), W.data_ptr(), None if R is None else R.data_ptr(),
                                   Y.data_ptr(), M, K, N, int(w16), o, sp)

        def sample(n, flush_between):
            """n launches queued back to back (a flush kernel between them
            when cold), each timed by its own event pair."""
            return queued_launch_times(launch, n, (lambda: flush.fill_(1.0)) if flush_between else None)

        # warm up for a fixed time, not a count, so the clocks have ramped
        # after the host-side input generation whatever the kernel's length
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            for _ in range(10):
                assert launch() == 0
            torch.cuda.synchronize()
        n = 100 if M * N * K < 1e11 else 30
        warm = sample(n, False)
        flops = 2 * M * N * K
        abytes = M * K * (8 if swiglu else 4) + K * N * (2 if w16 else 4) + M * N * 4 * (2 if R is not None else 1)
        row = {"config": name, "M": M, "K": K, "N": N, "tile": binding.kernel_config(M, K, N, swiglu=swiglu, w16=w16),
               "warm_median_us": round(float(np.median(warm)), 2), "warm_min_us": round(float(warm.min()), 2),
               "warm_p90_us": round(float(np.percentile(warm, 90)), 2),
               "tflops": round(flops / np.median(warm) / 1e6, 2),
               "frac_fp32_mfma_peak": round(flops / np.median(warm) / 1e6 / PEAK_FP32_MFMA_TFLOPS, 4)}
        if cold:
            cm = float(np.median(sample(n, True)))
            row["cold_median_us"] = round(cm, 2)
            row["cold_alg_GBps"] = round(abytes / cm / 1e3, 1)
        if name.startswith("cfg1"):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(1000):
                launch()
            torch.cuda.synchronize()
            row["amortised_us_per_launch"] = round((time.perf_counter() - t0) / 1000 * 1e6, 2)
        # context: the plain fp32 product in torch (hipBLASLt); no SwiGLU, no residual
        A = (torch.nn.functional.silu(G) * U) if swiglu else X
        Wf = W.float()
        Yt = torch.empty_like(Y)
        for _ in range(5):
            torch.matmul(A, Wf, out=Yt)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            torch.matmul(A, Wf, out=Yt)
        torch.cuda.synchronize()
        row["torch_matmul_fp32_us"] = round((time.perf_counter() - t0) / n * 1e6, 2)
        rows_out.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del Y, Yt, A
    hdr = ("| config | M×K×N | tile | warm median µs | min | p90 | TFLOP/s | % of 157.3 | cold µs | cold GB/s | "
           "torch.matmul fp32 µs (plain product) |")
    print(hdr)
    print("|" + "---|" * 11)
    for r in rows_out:
        print(f"| {r['config']} | {r['M']}×{r['K']}×{r['N']} | {r['tile']} | {r['warm_median_us']} | {r['warm_min_us']} | "
              f"{r['warm_p90_us']} | {r['tflops']} | {r['frac_fp32_mfma_peak'] * 100:.1f} | {r.get('cold_median_us', '')} | "
              f"{r.get('cold_alg_GBps', '')} | {r['torch_matmul_fp32_us']} |")
    c1 = next(r for r in rows_out if r["config"].startswith("cfg1"))
    print(f"\ncfg1 amortised over 1000 back-to-back launches: {c1['amortised_us_per_launch']} us per launch")


SHARDS = [
    # product, M, K, N, sharded dimension, swiglu, w16, residual
    ("lm_head, 16 x 512 tokens", 8192, 768, 50304, "N", False, True, False),
    ("lm_head, seq 512", 512, 768, 16384, "N", False, True, False),
    ("ffn_gate_up, 16 x 512 tokens", 8192, 768, 3072, "N", False, True, False),
    ("ffn_down SwiGLU, 16 x 512 tokens", 8192, 3072, 768, "K", True, True, True),
    ("ffn_down SwiGLU, seq 512 (fp32 W)", 512, 3072, 768, "K", True, False, True),
]


def time_shards():
    """Each product at the shape one GPU holds when it is sharded over g GPUs
    without changing the kernel: column-parallel weights split N, and the
    down-projection, whose G and U arrive split along d_ff, splits K (its
    partial outputs would then be summed across GPUs, which is not timed
    here).  Per launch, events recorded by the launch itself, as for the
    workload configurations; the last column compares g shards' time with
    the whole product's: t(1) / (g t(g))."""
    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding, inputs
    lib = binding.load_library()
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    sp = st.cuda_stream
    lines = ["| product | GPUs | shard M×K×N | tile | warm median µs | TFLOP/s | % of 157.3 | t(1) / (g·t(g)) |",
             "|---|---|---|---|---|---|---|---|"]
    for seed, (name, M0, K0, N0, dim, swiglu, w16, resid) in enumerate(SHARDS):
        t1 = None
        for g in (1, 2, 4, 8):
            M, K, N = M0, (K0 // g if dim == "K" else K0), (N0 // g if dim == "N" else N0)
            c = inputs.random_case(900 + seed, M, K, N, swiglu=swiglu, w16=w16, residual=resid)
            d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in c.items()}
            Y = torch.empty((M, N), device=dev)
            R = d.get("R")

            wsb = lib.gemm_fwd_workspace_bytes(M, K, N, int(swiglu), int(w16), -1)
            ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)

            def launch(ev=(None, None)):
                o = binding.opts(-1, ws.data_ptr() if wsb else None, wsb, *ev)
                if swiglu:
                    return lib.gemm_fwd_swiglu_ex(d["G"].data_ptr(), d["U"].data_ptr(), d["W"].data_ptr(),
                                                  R.data_ptr(), Y.data_ptr(), M, K, N, int(w16), o, sp)
                return lib.gemm_fwd_ex(d["X"].data_ptr(), d["W"].data_ptr(), None if R is None else R.data_ptr(),
                                       Y.data_ptr(), M, K, N, int(w16), o, sp)

            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.2:
                for _ in range(10):
                    assert launch() == 0
                torch.cuda.synchronize()
            n = 30 if M * N * K > 1e11 else 100
            us = float(np.median(queued_launch_times(launch, n)))
            t1 = us if g == 1 else t1
            tf = 2 * M * N * K / us / 1e6
            tile = binding.kernel_config(M, K, N, swiglu=swiglu, w16=w16)
            lines.append(f"| {name} | {g} | {M}×{K}×{N} | {tile} | {us:.2f} | {tf:.1f} | "
                         f"{100 * tf / PEAK_FP32_MFMA_TFLOPS:.1f} | {t1 / (g * us):.2f} |")
            print(lines[-1], file=sys.stderr, flush=True)
            del d, Y, R
    print("\n".join(lines))


def main():
    args = parse()
    if args.shards:
        time_shards()
        return
    if args.configs:
        import torch
        torch.backends.cuda.matmul.allow_tf32 = False
        time_configs()
        return
    if args.counters_from or args.traffic_from:
        counters_from(args.counters_from, args.traffic_from)
        return
    if args.trace_from:
        trace_from(args.trace_from)
        return
    if args.counter_workloads:
        counter_workloads()
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.backward:
        time_backward()
        return
    if args.loss:
        time_loss()
        return
    if args.activation:
        time_activation()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "`bench.py --shards` times each product at the shape one GPU would hold", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from tiled_dense_gemm_matmul_amd import binding

    binding.load_library()
    dev = torch.device("cuda:0")
    cases = workload()

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    launches = []
    for name, c in cases:
        M, K, N = shape_of(c)
        W = d(c["W"])
        R = d(c["R"]) if "R" in c else None
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        w16 = c["W"].dtype == np.float16
        lib = binding.load_library()
        # split-K configurations take a workspace, allocated (zero-filled)
        # here, outside the timed region
        wsb = lib.gemm_fwd_workspace_bytes(M, K, N, int("G" in c), int(w16), -1)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
        if "G" in c:
            G, U = d(c["G"]), d(c["U"])
            keep = (G, U, W, R, Y, ws)
            args_ = (G.data_ptr(), U.data_ptr(), W.data_ptr(), R.data_ptr(), Y.data_ptr(), M, K, N,
                     binding.GEMM_W_F16 if w16 else binding.GEMM_W_F32)
            fn = lib.gemm_fwd_swiglu_ex
            cfg = binding.kernel_config(M, K, N, swiglu=True, w16=w16)
        else:
            X = d(c["X"])
            keep = (X, W, R, Y, ws)
            args_ = (X.data_ptr(), W.data_ptr(), None if R is None else R.data_ptr(), Y.data_ptr(), M, K, N,
                     binding.GEMM_FLAG_W_F16 if w16 else 0)
            fn = lib.gemm_fwd_ex
            cfg = binding.kernel_config(M, K, N, swiglu=False, w16=w16)
        plain = binding.opts(-1, ws.data_ptr() if wsb else None, wsb)
        launches.append({"name": name, "fn": fn, "args": args_, "keep": keep, "M": M, "K": K, "N": N,
                         "ws": (ws.data_ptr() if wsb else None, wsb), "plain": plain, "workspace_bytes": wsb,
                         "flops": 2 * M * N * K, "w16": w16, "config": cfg,
                         "bytes": (M * K * (8 if "G" in c else 4) + K * N * (2 if w16 else 4)
                                   + M * N * 4 * (2 if R is not None else 1))})
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    dom_idx = next(i for i, L in enumerate(launches) if L["name"] == "lm_head")

    def step(events=None, which=()):
        for i, L in enumerate(launches):
            if events is not None and i in which:
                # the library records the pair at the kernel's own start and end
                e0, e1 = events[i]
                st = L["fn"](*L["args"], binding.opts(-1, *L["ws"], e0.handle, e1.handle), sp)
            else:
                st = L["fn"](*L["args"], L["plain"], sp)
            if st != 0:
                raise RuntimeError(f"{L['name']}: {binding.status_string(st)}")

    def new_events(n):
        # the library's timing events: recording them writes back and
        # invalidates no caches, so the timed kernel and the launches after
        # it run as they do untimed
        return [[[binding.TimingEvent(), binding.TimingEvent()] for _ in launches] for _ in range(n)]

    # The events of the timed region and of the per-kernel pass are made
    # first: making thousands of them takes the host milliseconds, during
    # which the GPU would idle and its clock drop just before the timed steps.
    ev = new_events(args.steps)
    nb = min(args.steps, 50)
    evb = new_events(nb)
    torch.cuda.synchronize()

    # Time-based pre-warm, then the counted warm-up.  After the host has spent
    # seconds generating inputs the engine clock starts low and ramps within
    # a few hundred milliseconds of sustained work; a handful of counted
    # warm-up steps (about a millisecond) does not reach steady state.
    prewarm_steps = 0
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_s:
        for _ in range(20):
            step()
        prewarm_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: whole steps, events around the dominant kernel only
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s], (dom_idx,))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = [ev[s][dom_idx][0].elapsed_ms(ev[s][dom_idx][1]) for s in range(args.steps)]

    # per-kernel breakdown (not timed as steps): events around every launch
    for s in range(nb):
        step(evb[s], range(len(launches)))
    torch.cuda.synchronize()

    step_flops = sum(L["flops"] for L in launches)
    ms_per_step = wall / args.steps * 1e3
    kernels = {}
    for i, L in enumerate(launches):
        ms = [evb[s][i][0].elapsed_ms(evb[s][i][1]) for s in range(nb)]
        avg_us = float(np.mean(ms)) * 1e3
        kernels[L["name"]] = {
            "M": L["M"], "K": L["K"], "N": L["N"], "w": "f16" if L["w16"] else "f32",
            "config": L["config"], "workspace_bytes": L["workspace_bytes"], "avg_us": round(avg_us, 3),
            "median_us": round(float(np.median(ms)) * 1e3, 3),
            "tflops": round(L["flops"] / avg_us / 1e6, 3),
            "frac_fp32_mfma_peak": round(L["flops"] / avg_us / 1e6 / PEAK_FP32_MFMA_TFLOPS, 4),
            "alg_GBps": round(L["bytes"] / avg_us / 1e3, 1),
        }

    dom = launches[dom_idx]
    dom_avg_us = float(np.mean(dom_ms)) * 1e3
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_sha256_16") == kernel_hash() and t.get("tile") == dom["config"] == LM_HEAD_TILE:
            traffic = t.get("bytes_per_launch")
    achieved = dom["flops"] / dom_avg_us / 1e6
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4), "traffic": traffic,
        "kernel": "lm_head (matmul_w16 512x768x16384)", "avg_us": round(dom_avg_us, 3),
        "launches": args.steps,
    }

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cases, args.cpu_seconds)

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_s": args.prewarm_s,
        "prewarm_steps": prewarm_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "seq512 forward GEMM family: qkvo_residual + qkvo (512x768x768 f32 W), "
                        "ffn_down swiglu (512x3072x768 f32 W, +R), ffn_gate_up (512x768x3072 f16 W), "
                        "lm_head (512x768x16384 f16 W)",
            "step_gflop": round(step_flops / 1e9, 4),
            "frac_fp32_mfma_peak": round(value / PEAK_FP32_MFMA_TFLOPS, 4),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernels_note": "per-kernel HIP-event durations (the library's timing events, recorded by the launch "
                        "at kernel start and end) "
                        f"from a separate pass of {min(args.steps, 50)} steps",
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
