"""Host logic of bench.py, on the CPU: the one-GPU guard, the kernel lists of
its counter sets against the inputs it launches, and the summaries it writes
from rocprofv3 output (counters, HBM traffic, kernel trace), fed with
synthetic CSV files whose figures are known."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_step_counter_set_matches_the_step():
    specs = bench.COUNTER_SETS["step"]["kernels"]
    assert [s[0] for s in specs] == bench.STEP_LABELS
    for (label, case), (name, M, K, N, swiglu, w16, resid) in zip(bench.workload(), specs):
        assert label == name
        assert bench.shape_of(case) == (M, K, N)
        assert ("G" in case, case["W"].dtype.itemsize == 2, "R" in case) == (swiglu, w16, resid)


def test_workload_counter_set_matches_its_inputs():
    from tiled_dense_gemm_matmul_amd import inputs
    gens = {g: getattr(inputs, g)() for g in {w[0] for w in bench.WORKLOADS}}
    for (gen, keys, rows), (name, M, K, N, swiglu, w16, resid) in zip(bench.WORKLOADS,
                                                                       bench.COUNTER_SETS["workloads"]["kernels"]):
        c = gens[gen]
        A = c[keys[0]]
        W = c[keys[2] if swiglu else keys[1]]
        assert (rows or A.shape[0], A.shape[1], W.shape[1]) == (M, K, N), name
        assert (len(keys) == 4, W.dtype.itemsize == 2, (keys[3] if swiglu else keys[2]) is not None) == \
               (swiglu, w16, resid), name


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


DUR_US = 10.0          # under 50 us: no clock shown
CLOCK_MHZ = 2000.0


def _counter_value(counter, M, K, N):
    mfma = 2 * M * K * N / 2048
    return {
        "SQ_INSTS_MFMA": mfma, "SQ_INSTS_VALU": 2 * mfma, "SQ_INSTS_LDS": 0.25 * mfma,
        "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * 2400 * DUR_US, "GRBM_GUI_ACTIVE": 8 * CLOCK_MHZ * DUR_US,
        "SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 10.0, "TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0,
        "SQ_VALU_MFMA_COEXEC_CYCLES": 0.0,
    }.get(counter, 7.0)


def _counter_run(path, specs, counters, rounds=2, value=None):
    rows, disp = [], 1
    for _ in range(rounds):
        # a kernel outside the library between rounds must be ignored
        rows.append({"Dispatch_Id": disp, "Kernel_Name": "void fill_kernel<float>(float*)", "Counter_Name": counters[0],
                     "Counter_Value": 1e9, "Start_Timestamp": 0, "End_Timestamp": 1})
        disp += 1
        for (name, M, K, N, *_r) in specs:
            for ctr in counters:
                v = value(ctr, name, M, K, N) if value else _counter_value(ctr, M, K, N)
                rows.append({"Dispatch_Id": disp, "Kernel_Name": f"void gemm_fwd_kernel<Tile<{M}>>(Params)",
                             "Counter_Name": ctr, "Counter_Value": v, "Start_Timestamp": 1000 * disp,
                             "End_Timestamp": 1000 * disp + int(DUR_US * 1000)})
            disp += 1
    _write_csv(os.path.join(path, "pmc", "pmc_counter_collection.csv"), rows)


def test_counter_and_traffic_summaries(tmp_path):
    cbase, tbase, out = tmp_path / "counters", tmp_path / "traffic", tmp_path / "out"
    out.mkdir()
    for set_name, cs in bench.COUNTER_SETS.items():
        for run, ctrs in bench.COUNTER_PASSES.items():
            _counter_run(str(cbase / set_name / run), cs["kernels"], ctrs.split())
        # fetched bytes = the algorithmic reads, written bytes = twice the algorithmic writes
        _counter_run(str(tbase / set_name / "fetch"), cs["kernels"], ["FETCH_SIZE"],
                     value=lambda c, n, M, K, N, cs=cs: (
                         bench.alg_bytes(M, K, N, *next(k[4:] for k in cs["kernels"] if k[0] == n)) - M * N * 4)
                     / 2 / 1024)
        _counter_run(str(tbase / set_name / "write"), cs["kernels"], ["WRITE_SIZE"],
                     value=lambda c, n, M, K, N: 2 * M * N * 4 / 1024)
    for run, kib in (("copy_fetch", bench.COPY_BYTES / 2 / 1024), ("copy_write", bench.COPY_BYTES / 1024)):
        _write_csv(str(tbase / run / "pmc" / "pmc_counter_collection.csv"),
                   [{"Dispatch_Id": i, "Kernel_Name": "void at::native::copy_kernel(...)", "Counter_Name": "X",
                     "Counter_Value": kib, "Start_Timestamp": 0, "End_Timestamp": 1} for i in range(5)])
    bench.counters_from(str(cbase), str(tbase), out_dir=str(out))
    step = (out / "seq512_counters.md").read_text()
    # durations under 50 us show no clock
    assert "| qkvo | 512×768×768 | 2 | 10.0 | — | 1.000 | 50.0% | 1.00 | 0 | 0.250 | 10.0% | 75.0% |" in step
    assert "| lm_head | 512×768×16384 | 2 |" in step
    work = (out / "workload_counters.md").read_text()
    assert "| cfg5b lm_head, M=8191 | 8191×768×50304 | 2 | 10.0 | — | 1.000 | 50.0% |" in work
    traffic = (out / "seq512_traffic.md").read_text()
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in traffic
    for line in traffic.splitlines():
        if line.startswith("| ffn_down"):
            assert line.rstrip().endswith("| 1.00 | 2.00 |"), line
    lm = json.loads((out / "lm_head_traffic.json").read_text())
    reads = 512 * 768 * 4 + 768 * 16384 * 2
    assert lm["fetch_bytes"] == reads and lm["write_bytes"] == 2 * 512 * 16384 * 4
    assert lm["bytes_per_launch"] == lm["fetch_bytes"] + lm["write_bytes"]
    assert lm["kernel_sha256_16"] == bench.kernel_hash()
    assert (out / "workload_traffic.md").exists()


def test_kernel_trace_summary(tmp_path):
    pre, warm, steps = 7, 2, 4
    nb = min(steps, 50)
    n = len(bench.STEP_LABELS)
    rows, disp = [], 1
    for s in range(pre + warm + steps + nb):
        timed = pre + warm <= s < pre + warm + steps
        rows.append({"Dispatch_Id": disp, "Kernel_Name": "void fill_kernel(float*)", "Start_Timestamp": 0,
                     "End_Timestamp": 5})
        disp += 1
        for i in range(n):
            us = (10.0 * (i + 1)) if timed else 1.0
            rows.append({"Dispatch_Id": disp, "Kernel_Name": f"void gemm_fwd_kernel<{i}>(Params)",
                         "Start_Timestamp": 1000 * disp, "End_Timestamp": 1000 * disp + int(us * 1000)})
            disp += 1
    _write_csv(str(tmp_path / "trace" / "b" / "bench_kernel_trace.csv"), rows)
    line = {"steps": steps, "warmup": warm, "prewarm_steps": pre, "ms_per_step": 0.2, "value": 95.0,
            "roofline": {"avg_us": 50.1}, "kernels": {k: {"avg_us": 1.1} for k in bench.STEP_LABELS}}
    (tmp_path / "bench.log").write_text("noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "out"
    out.mkdir()
    bench.trace_from(str(tmp_path), out_dir=str(out))
    md = (out / "seq512_step_kernel_trace.md").read_text()
    assert "| lm_head | 4 | 50.00 | 50.00 | 50.00 |" in md
    assert "| qkvo_residual | 4 | 10.00 |" in md
    assert f"| 38.4 | {pre + warm + steps + nb} | 3.12 | 1.00 | 1.10 |" in md   # qkvo_residual, all launches
    assert "against 50.00 us by the trace over the same launches" in md
    plain = dict(line, value=120.0, roofline={"avg_us": 51.0, "launches": steps, "frac": 0.5})
    (tmp_path / "bench_plain.log").write_text(json.dumps(plain) + "\n")
    bench.trace_from(str(tmp_path), out_dir=str(out))
    md = (out / "seq512_step_kernel_trace.md").read_text()
    assert "lm_head averaged 51.0 us by HIP events over its 4 timed-region launches (+2.0% against the trace" in md
    # a trace with a launch missing is refused
    _write_csv(str(tmp_path / "trace" / "b" / "bench_kernel_trace.csv"), rows[:-1])
    with pytest.raises(SystemExit):
        bench.trace_from(str(tmp_path), out_dir=str(out))
