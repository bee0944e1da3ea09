"""Benchmark of the quantized-state decode step on one MI355X.

A step is one qstate_decode_step over the whole batch: dequantize, decay +
update, readout and requantize of every (b, h) state.  Default workload:
Mamba2 scalar decay, B=256, H=32, head_dim 64 x d_state 128, 8 of 32 heads in
bf16 (slowest decay), the rest int8 with value-axis scales and Philox
stochastic rounding.

Cold mode (default) rotates enough replicas of the state that the working
set (>= 512 MB) cannot stay in the 256 MB Infinity Cache, so every step
streams its state from HBM; hot mode reuses one state.  Inputs are resident
in HBM before timing (a pool of distinct steps, rotated).  Timing: HIP
events on the stream the kernels are launched on, around exactly --steps
launches after --warmup untimed ones.

Prints one JSON line (see the keys in main()).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak
METRIC = "quantized-state decode steps/sec and state GB/s (% HBM peak) at B=256, 1 GPU"
CSRC = os.path.join(ROOT, "quantized_recurrent_state_qstate_amd", "csrc")


def kernel_hash() -> str:
    """Hash of the device sources: counter-derived traffic is valid only for these."""
    import glob
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, m) -> dict:
    """Bytes one step must move, from the documented storage format:
    the stored state read and written once, the inputs read, the outputs written."""
    import numpy as np
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    if w.map_mode == "none":
        prot = np.zeros((H, dk), bool)
    elif w.map_mode == "head":
        prot = np.repeat(np.asarray(m, bool)[:, None], dk, axis=1)
    else:
        prot = np.asarray(m, bool).reshape(H, dk)
    nhp = prot.sum(1)
    nq = dk - nhp
    hpb = 4 if w.hp_dtype == "fp32" else 2
    codes = B * int(sum(dv * (((int(n) * w.qbits + 7) // 8 + 3) // 4 * 4) for n in nq))   # rows padded to 4 B
    scales = B * int(sum(dv * 4 for n in nq if n > 0))
    hp = B * int(sum(dv * ((int(n) * hpb + 3) // 4 * 4) for n in nhp))
    state_rw = 2 * (codes + scales + hp)
    if w.lrb_rank:
        r = w.lrb_rank
        state_rw += B * H * (dv * r * 4 + 2 * dk * r * 4 + 2 * 4)   # W read, U and n read+write
    inb = 2 if w.in_dtype == "bf16" else 4
    decay = B * H * (dk if w.decay_mode == "key" else 1) * 4
    beta = B * H * 4 if w.has_beta else 0
    inputs = B * H * (2 * dk + dv) * inb + decay + beta
    outputs = B * H * dv * 4
    return {"state_rw": state_rw, "state": state_rw // 2, "inputs": inputs, "outputs": outputs,
            "total": state_rw + inputs + outputs}


def lib_config(w, m):
    from quantized_recurrent_state_qstate_amd import StateConfig
    return StateConfig(kind=w.kind, decay_mode=w.decay_mode, B=w.B, H=w.H, dk=w.dk, dv=w.dv, qbits=w.qbits,
                       hp_dtype=w.hp_dtype, map_mode=w.map_mode, map=m, in_dtype=w.in_dtype,
                       rounding=w.rounding, sr_bits=w.sr_bits, bdr=w.bdr, lrb_rank=w.lrb_rank,
                       lrb_period=w.lrb_period, lrb_theta=w.lrb_theta, seed=w.philox_seed)


def cpu_baseline(w, m, budget_s: float) -> dict:
    """The oracle as it stands (single-threaded C), timed on this host on whole
    batch elements of the same workload; scaled to full-batch steps/s."""
    import numpy as np
    import oracle
    per_b = w.H
    bs = 1
    ocfg = oracle.Cfg(kind=w.kind, decay_mode=w.decay_mode, B=bs, H=w.H, dk=w.dk, dv=w.dv, qbits=w.qbits,
                      hp_dtype=w.hp_dtype, map_mode=w.map_mode, map=m,
                      rounding="rtn" if w.rounding == "nearest" else "sr", sr_bits=w.sr_bits, bdr=w.bdr,
                      lrb_rank=w.lrb_rank, lrb_period=w.lrb_period, lrb_theta=w.lrb_theta,
                      seed=w.philox_seed)

    def run(nb, nsteps=1):
        ocfg.B = nb
        rng = np.random.default_rng(0)
        st = oracle.new_state(ocfg)
        oracle.quantize(ocfg, rng.standard_normal((nb, w.H, w.dv, w.dk)).astype(np.float32), st, 0)
        t = 0.0
        for s in range(1, nsteps + 1):
            inp = w.step_inputs(s, B=nb)
            f = {k: (None if v is None else v.float().numpy()) for k, v in inp.items()}
            t0 = time.perf_counter()
            oracle.step(ocfg, st, **f, step=s)
            t += time.perf_counter() - t0
        return t

    t1 = run(1)
    nb = max(1, min(w.B, int(budget_s / max(t1, 1e-6))))
    # whole batches: as many consecutive steps as fit the budget
    nsteps = 1 if nb < w.B else max(1, int(budget_s / max(t1 * w.B, 1e-6)))
    t = run(nb, nsteps)
    sec_per_step = t / (nb * nsteps) * w.B
    return {"value": 1.0 / sec_per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{nb} of {w.B} batch elements ({nb * per_b} heads) x {nsteps} step(s), {t:.1f} s "
                      f"of oracle step time; single-threaded C oracle on "
                      f"{platform.processor() or platform.machine()}, {os.cpu_count()} host threads visible"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="mamba2")
    ap.add_argument("--mode", choices=["cold", "hot"], default="cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true", help="replay the launches as one captured HIP graph")
    ap.add_argument("--sr-bits", type=int, default=0, help="override the workload's random bits per element")
    ap.add_argument("--rounding", choices=["nearest", "stochastic"], default=None,
                    help="override the workload's rounding mode")
    ap.add_argument("--map-frac", type=float, default=None,
                    help="override the fraction of protected heads or channels")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one device copy of this size (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode step needs no inter-GPU exchange and this build "
              "runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_recurrent_state_qstate_amd import QState, _lib, build_map
    from quantized_recurrent_state_qstate_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.sr_bits:
        w = w.scaled(sr_bits=args.sr_bits)
    if args.rounding:
        w = w.scaled(rounding=args.rounding)
    if args.map_frac is not None:
        w = w.scaled(map_frac=args.map_frac)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    m = None
    if w.map_stat() is not None:
        stat, groups, per = w.map_stat()
        m = build_map(stat, groups, per, w.map_frac)
    qs = QState(lib_config(w, m))
    L = _lib.lib()
    alg = algorithmic_bytes(w, m)
    resident = sum(qs.sizes.values())

    R = 1 if args.mode == "hot" else max(2, math.ceil(512e6 / resident))
    states = [qs.new_state() for _ in range(R)]
    g = torch.Generator(device=dev).manual_seed(12345)
    S0 = torch.randn(w.B, w.H, w.dv, w.dk, generator=g, device=dev)
    for st in states:
        qs.quantize(S0, st, step=0)
    del S0
    P = 16
    pool = []
    for t in range(P):
        inp = w.step_inputs(t)
        pool.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    out = torch.empty(w.B, w.H, w.dv, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    tens = [qs._tensors(st) for st in states]
    ins = [_lib.Inputs(p["q"].data_ptr(), p["k"].data_ptr(), p["v"].data_ptr(), p["decay"].data_ptr(),
                       None if p["beta"] is None else p["beta"].data_ptr()) for p in pool]
    tref = [ctypes.byref(t) for t in tens]
    iref = [ctypes.byref(i) for i in ins]
    h = qs._h
    optr = out.data_ptr()
    step_fn = L.qstate_decode_step

    def enqueue(i0, n, stream_ptr):
        bad = 0
        for i in range(i0, i0 + n):
            bad |= step_fn(h, tref[i % R], iref[i % P], optr, i, stream_ptr)
        return bad

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    if enqueue(0, args.warmup, sp):
        _lib.check(-4, "warmup")
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        G = math.lcm(R, P)
        G = G * max(1, 64 // G)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                if enqueue(args.warmup, G, torch.cuda.current_stream().cuda_stream):
                    _lib.check(-4, "capture")
        torch.cuda.synchronize()
        reps = max(1, args.steps // G)
        args.steps = reps * G
        graph.replay()
        torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    e0.record(stream)
    if graph is not None:
        for _ in range(reps):
            graph.replay()
        bad = 0
    else:
        bad = enqueue(args.warmup, args.steps, sp)
    e1.record(stream)
    c1 = time.perf_counter()
    torch.cuda.synchronize()
    if bad:
        _lib.check(-4, "timed steps")
    ms_total = e0.elapsed_time(e1)
    ms = ms_total / args.steps
    steps_per_s = 1e3 / ms
    state_gbps = alg["state_rw"] / (ms * 1e-3) / 1e9
    achieved = alg["total"] / (ms * 1e-3) / 1e9

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    traffic = None
    pmc_path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(pmc_path):
        with open(pmc_path) as f:
            rec = json.load(f)
        if rec.get("kernel_hash") == kernel_hash():
            traffic = rec.get("bytes_per_launch")

    res = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.recurrence}, B={w.B}, H={w.H}, dk={w.dk}, dv={w.dv}, "
                               f"{'int%d' % w.qbits}, map={w.map_mode}:{w.map_frac}, {w.rounding}"
                               + (f" {w.sr_bits}-bit" if w.rounding == "stochastic" else "")
                               + (", bdr" if w.bdr else "") + (f", lrb r={w.lrb_rank}" if w.lrb_rank else ""),
                   "state": "int%d codes" % w.qbits + ("" if w.map_mode == "none" else
                                                        f" + {w.hp_dtype} protected "
                                                        + ("heads" if w.map_mode == "head" else "key channels")),
                   "mode": args.mode, "replicas": R, "graph": bool(graph is not None),
                   "tokens_per_s": round(steps_per_s * w.B, 1)},
        "state_GBps": round(state_gbps, 1),
        "state_pct_hbm_peak": round(100.0 * state_gbps / PEAK_HBM_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": alg["total"], "kernel": qs.kernel_name},
        "host_enqueue_ms_per_step": round((c1 - c0) * 1e3 / args.steps, 4),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, m, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
