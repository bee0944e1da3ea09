"""Host logic of bench.py (no GPU): the trace summary's choice of the timed
launches, the one-GPU guard, the source hash that keys the traffic record,
and the algorithmic byte count of the headline workload."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _trace(tmp_path, durations, other=()):
    """A rocprofv3-style kernel_trace.csv: step-kernel launches with the given
    durations (ns), in launch order, plus other kernels."""
    d = tmp_path / "kt" / "host"
    d.mkdir(parents=True)
    rows, t = [], 1000
    for i, dur in enumerate(durations):
        rows.append({"Kernel_Name": "void qs::k_step_dense<8, 1>(qs::Args)", "Start_Timestamp": t,
                     "End_Timestamp": t + dur})
        t += dur + 100
    for name, dur in other:
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 100
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    return str(tmp_path / "kt")


def test_trace_summary_picks_the_timed_launches(tmp_path):
    # 10 prewarm + 4 warmup launches at 900 ns, 6 timed at 100..600 ns, 3 context launches at 5000
    durs = [900] * 14 + [100, 200, 300, 400, 500, 600] + [5000] * 3
    path = _trace(tmp_path, durs, other=[("qs::k_quantize(qs::Args)", 7000)])
    out = bench.trace_summary(path, 14, 6)
    line = [l for l in out.splitlines() if l.startswith("Headline run")][0]
    assert "launches 14 .. 19" in line
    assert "6 launches, average 350 ns, min 100 ns, max 600 ns" in line
    assert "k_quantize" in out                    # other kernels are listed, not counted as steps


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def test_kernel_hash_follows_the_dense_unit_sources():
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_hash("dense") == h
    assert bench.kernel_hash("lrb") != h          # another unit, other headers


def test_headline_algorithmic_bytes():
    from quantized_recurrent_state_qstate_amd import build_map
    from quantized_recurrent_state_qstate_amd.workloads import WORKLOADS
    w = WORKLOADS["mamba2"]
    stat, groups, per = w.map_stat()
    m = build_map(stat, groups, per, w.map_frac)
    alg = bench.algorithmic_bytes(w, m)
    B, H, dv, dk = w.B, w.H, w.dv, w.dk
    n16 = int(m.sum())                                     # bf16 heads per batch element
    state = B * ((H - n16) * (dv * dk + 4 * dv) + n16 * 2 * dv * dk)
    assert n16 == 8
    assert alg["state_rw"] == 2 * state == 170917888
    assert w.has_beta                                       # Mamba2: beta = dt
    inputs = B * H * ((2 * dk + dv) * 2 + 4 + 4)           # q, k, v in bf16; fp32 decay and beta
    outputs = B * H * dv * 4
    assert alg["total"] == 2 * state + inputs + outputs == 178323456
