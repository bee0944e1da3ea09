"""Synthetic state-error study of the quantized decode step (needs a GPU).

Runs a gated linear recurrence for T steps through libqstate under several
state formats and rounding modes, next to the same recurrence in float64,
and reports how the stored state drifts.  It reproduces on synthetic inputs
the qualitative claims of the pages' abstracts:

* "Quantizing Recurrent Language Models Is Easier Than You Think": error
  accumulates under repeated requantization and stochastic rounding counters
  it; scales grouped along the value axis match the output channels.
* "Preserving Updates in Low-Bit Recurrent State Quantization": small
  updates are lost at each requantization, the errors are coherent (they
  point the same way step after step), Bounded Directional Rounding rounds
  elements that would move against their update toward it, and the Low-Rank
  Bypass keeps the small updates until they are large enough to merge.

Metrics of one configuration (means over heads; steps after a warm-up):

  state_err   ||S_q - S_ref|| / ||S_ref|| at the last step, S_q the stored
              state as dequantized (with the bypass buffer), S_ref the exact
              float64 recurrence from the same inputs
  out_err     ||o_q - o_ref|| / ||o_ref|| at the last step
  retention   <R, D> / <D, D>: how much of a step's exact change D (from the
              stored state before the step) the stored state R realizes
  reversal    fraction of elements whose stored value moved against D
              (|D| above 1e-6 of the row's largest value)
  coherence   cosine between consecutive steps' rounding errors
              E_t = S_q,t - (exact step of S_q,t-1)

Scale grouping (value axis, key axis, one scale per head) runs through the
library's scale_axis; run_grouping is a float64 simulation of the same
quantizer, kept as an independent cross-check of the grouped path.

    python -m quantized_recurrent_state_qstate_amd.error_study [--T 256] [--json out.json]
    python -m quantized_recurrent_state_qstate_amd.error_study --horizons   # error after 64/256/1024 steps
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np


def _inputs(B, H, dk, dv, t, rp, seed):
    """Step t of a regime: q, k ~ N(0,1) * qk_scale and v ~ N(0,1), or, with
    persist p > 0, k = qk_scale (kbar + (1-p) eps) and v = sigma (vbar + (1-p)
    eps) around fixed per-(b,h) directions kbar, vbar, with per-value-channel
    magnitudes sigma spread log-normally over a factor vspread (fixed per
    head); decay sigmoid(N(mu, 1)) per key channel."""
    import torch
    g = torch.Generator().manual_seed(seed * 1_000_003 + t)
    p = rp.get("persist", 0.0)
    q = torch.randn(B, H, dk, generator=g) * rp["qk_scale"]
    k = torch.randn(B, H, dk, generator=g)
    v = torch.randn(B, H, dv, generator=g)
    if p > 0:
        gf = torch.Generator().manual_seed(seed + 17)
        kbar = torch.randn(B, H, dk, generator=gf)
        vbar = torch.randn(B, H, dv, generator=gf)
        sig = torch.exp(torch.rand(H, dv, generator=gf) * math.log(rp.get("vspread", 1.0)))
        k = kbar + (1.0 - p) * k
        v = sig[None] * (vbar + (1.0 - p) * v)
    k = k * rp["qk_scale"]
    a = torch.sigmoid(torch.randn(B, H, dk, generator=g) + rp["mu"])
    bf = torch.bfloat16
    return q.to(bf), k.to(bf), v.to(bf), a


def _initial_state(B, H, dk, dv, rp, seed):
    """fp32 initial state: zero, or init * N(0,1) scaled by the value
    channels' magnitudes (a long context already in the state)."""
    import torch
    if not rp.get("init", 0.0):
        return None
    gf = torch.Generator().manual_seed(seed + 17)
    torch.randn(B, H, dk, generator=gf)      # kbar, vbar, sigma: the stream of _inputs
    torch.randn(B, H, dv, generator=gf)
    sig = torch.exp(torch.rand(H, dv, generator=gf) * math.log(rp.get("vspread", 1.0)))
    g = torch.Generator().manual_seed(seed + 23)
    return rp["init"] * sig[None, :, :, None] * torch.randn(B, H, dv, dk, generator=g)


def _exact_step(S, q, k, v, a):
    """GLA step in float64: S <- S diag(a) + v k^T, o = S q (S[v][k])."""
    S = S * a[..., None, :] + v[..., :, None] * k[..., None, :]
    return S, (S * q[..., None, :]).sum(-1)


def run_library(cfgkw, B, H, dk, dv, T, rp, seed, warm, checkpoints=()):
    import torch

    from . import QState, StateConfig
    dev = torch.device("cuda")
    cfg = StateConfig(kind="additive", decay_mode="key", B=B, H=H, dk=dk, dv=dv, in_dtype="bf16", seed=7,
                      **cfgkw)
    qs = QState(cfg)
    st = qs.new_state()
    f64 = torch.float64
    S0 = _initial_state(B, H, dk, dv, rp, seed)
    if S0 is None:
        S_prev = torch.zeros(B, H, dv, dk, dtype=f64, device=dev)
    else:   # stored with the configuration's rounding; both runs start from the stored state
        qs.quantize(S0.to(dev).contiguous(), st)
        S_prev = qs.dequantize(st).to(f64)
    S_ref = S_prev.clone()
    ret, rev, coh = [], [], []
    E_prev = None
    o = o_ref = None
    at = {}

    def errors(S_q, o, S_ref, o_ref):
        nr = S_ref.norm(dim=(-1, -2)).clamp_min(1e-300)
        return dict(state_err=((S_q - S_ref).norm(dim=(-1, -2)) / nr).mean().item(),
                    out_err=((o.to(f64) - o_ref).norm(dim=-1) / o_ref.norm(dim=-1).clamp_min(1e-300)).mean().item())

    for t in range(T):
        q, k, v, a = (x.to(dev) for x in _inputs(B, H, dk, dv, t, rp, seed))
        o = qs.step(st, q, k, v, a, step=t + 1)
        qd, kd, vd, ad = (x.to(f64) for x in (q, k, v, a))
        S_ref, o_ref = _exact_step(S_ref, qd, kd, vd, ad)
        S_q = qs.dequantize(st).to(f64)
        S_pre, _ = _exact_step(S_prev, qd, kd, vd, ad)       # exact step of the stored state
        if t >= warm:
            D = S_pre - S_prev
            R = S_q - S_prev
            E = S_q - S_pre
            big = D.abs() > 1e-6 * S_pre.abs().amax(-1, keepdim=True)
            dd = (D * D).sum((-1, -2))
            ret.append(((R * D).sum((-1, -2)) / dd.clamp_min(1e-300)).mean().item())
            rev.append((((R * D) < 0) & big).sum().item() / max(int(big.sum().item()), 1))
            if E_prev is not None:
                num = (E * E_prev).sum((-1, -2))
                den = (E.norm(dim=(-1, -2)) * E_prev.norm(dim=(-1, -2))).clamp_min(1e-300)
                coh.append((num / den).mean().item())
            E_prev = E
        S_prev = S_q
        if t + 1 in checkpoints:
            at[t + 1] = errors(S_q, o, S_ref, o_ref)
    e = errors(S_prev, o, S_ref, o_ref)
    qs.close()
    return dict(state_err=e["state_err"], out_err=e["out_err"],
                retention=float(np.mean(ret)) if ret else float("nan"),
                reversal=float(np.mean(rev)) if rev else float("nan"),
                coherence=float(np.mean(coh)) if coh else float("nan"), at=at)


def run_grouping(grouping, qbits, rounding, B, H, dk, dv, T, rp, seed):
    """Float64 simulation: the exact step of the stored state, then
    quantization with one scale per row (value axis), per column (key axis)
    or per head; nearest or stochastic rounding."""
    import torch
    dev = torch.device("cuda")
    f64 = torch.float64
    Q = 127.0 if qbits == 8 else 7.0
    g = torch.Generator(device=dev).manual_seed(seed + 99)
    S0 = _initial_state(B, H, dk, dv, rp, seed)

    def quant(S_pre):
        if grouping == "value":
            m = S_pre.abs().amax(-1, keepdim=True)
        elif grouping == "key":
            m = S_pre.abs().amax(-2, keepdim=True)
        else:
            m = S_pre.abs().amax((-1, -2), keepdim=True)
        s = m / Q
        x = torch.where(s > 0, S_pre / torch.where(s > 0, s, 1.0), torch.zeros_like(S_pre))
        if rounding == "nearest":
            c = torch.round(x)
        else:
            c = torch.floor(x + torch.rand(x.shape, generator=g, device=dev, dtype=f64))
        return c.clamp(-Q, Q) * s

    S = torch.zeros(B, H, dv, dk, dtype=f64, device=dev) if S0 is None else quant(S0.to(dev).to(f64))
    S_ref = S.clone()
    for t in range(T):
        q, k, v, a = (x.to(dev).to(f64) for x in _inputs(B, H, dk, dv, t, rp, seed))
        S_ref, _ = _exact_step(S_ref, q, k, v, a)
        S_pre, _ = _exact_step(S, q, k, v, a)
        S = quant(S_pre)
    nr = S_ref.norm(dim=(-1, -2)).clamp_min(1e-300)
    return ((S - S_ref).norm(dim=(-1, -2)) / nr).mean().item()


LIB_CONFIGS = [
    ("int8 nearest", dict(qbits=8, rounding="nearest")),
    ("int8 SR16", dict(qbits=8, rounding="stochastic", sr_bits=16)),
    ("int4 nearest", dict(qbits=4, rounding="nearest")),
    ("int4 SR16", dict(qbits=4, rounding="stochastic", sr_bits=16)),
    ("int4 SR8", dict(qbits=4, rounding="stochastic", sr_bits=8)),
    ("int4 nearest+BDR", dict(qbits=4, rounding="nearest", bdr=True)),
    ("int4 nearest+BDR+LRB r8", dict(qbits=4, rounding="nearest", bdr=True, lrb_rank=8, lrb_period=64,
                                      lrb_theta=0.5)),
]


# Regimes: i.i.d. updates under a mean decay per step sigmoid(mu) = 0.95,
# 0.993, 0.999 (state memory about 20, 150 and 1000 steps); and structured
# updates closer to a language model's: persistent key and value directions,
# value channels whose magnitudes spread over a factor 10, and a long context
# already in the state, so each step's update is small against the state.
REGIMES = [
    ("fast decay, i.i.d. updates", dict(mu=3.0, qk_scale=1.0)),
    ("slow decay, i.i.d. updates", dict(mu=5.0, qk_scale=1.0)),
    ("very slow decay, i.i.d. updates", dict(mu=7.0, qk_scale=1.0)),
    ("very slow decay, persistent small updates", dict(mu=7.0, qk_scale=0.3, persist=0.7, vspread=10.0,
                                                       init=20.0)),
]


def study(B=16, H=4, dk=128, dv=128, T=256, seed=2024, warm=16, regimes=None, groupings=True):
    out = []
    for rname, rp in (regimes or REGIMES):
        rows = []
        for name, kw in LIB_CONFIGS:
            r = run_library(kw, B, H, dk, dv, T, rp, seed, warm)
            r["config"] = name
            rows.append(r)
        groups = []
        if groupings:
            # through the library's scale_axis: rows (value axis), key
            # channels, one per head
            for qbits in (8, 4):
                for rounding in ("nearest", "stochastic"):
                    e = {g: run_library(dict(qbits=qbits, rounding=rounding, scale_axis=g), B, H, dk, dv, T, rp,
                                        seed, warm)["state_err"] for g in ("value", "key", "head")}
                    groups.append(dict(qbits=qbits, rounding=rounding, **e))
        out.append(dict(regime=rname, decay=f"sigmoid(N({rp['mu']},1)) per key", params=rp,
                        library=rows, grouping=groups))
    return dict(setup=dict(B=B, H=H, dk=dk, dv=dv, T=T, inputs="bf16, see _inputs",
                           seed=seed, warm=warm), regimes=out)


HORIZON_CONFIGS = [
    ("int8 SR16", dict(qbits=8, rounding="stochastic", sr_bits=16)),
    ("int4 SR16", dict(qbits=4, rounding="stochastic", sr_bits=16)),
    ("int4 nearest", dict(qbits=4, rounding="nearest")),
    ("int4 nearest+BDR+LRB r8", dict(qbits=4, rounding="nearest", bdr=True, lrb_rank=8, lrb_period=64,
                                      lrb_theta=0.5)),
]


def horizon_study(B=16, H=4, dk=128, dv=128, horizons=(64, 256, 1024), seed=2024, regime=None):
    """Error after 64, 256 and 1024 decode steps from the same start (one run
    per configuration, read at each horizon): how a low-precision state fares
    on short decode horizons ("lower effective precision on shorter decode
    horizons", abstract of "Quantizing Recurrent Language Models Is Easier
    Than You Think").  Default regime: i.i.d. updates under very slow decay
    from an empty state, where the state keeps growing and each step's
    rounding error adds to the last (under the structured regime the error
    of a large stored context saturates within the first steps instead)."""
    rname, rp = regime or REGIMES[2]
    T = max(horizons)
    rows = []
    for name, kw in HORIZON_CONFIGS:
        r = run_library(kw, B, H, dk, dv, T, rp, seed, warm=T, checkpoints=set(horizons))
        rows.append(dict(config=name, at={h: r["at"][h] for h in horizons}))
    return dict(regime=rname, params=rp, horizons=list(horizons), rows=rows,
                setup=dict(B=B, H=H, dk=dk, dv=dv, seed=seed))


def horizon_markdown(res) -> str:
    hs = res["horizons"]
    out = [f"**{res['regime']}**: state error / output error after T decode steps", "",
           "| configuration | " + " | ".join(f"T = {h}" for h in hs) + " |",
           "|---|" + "---:|" * len(hs)]
    for r in res["rows"]:
        out.append(f"| {r['config']} | " + " | ".join(
            f"{r['at'][h]['state_err']:.3f} / {r['at'][h]['out_err']:.3f}" for h in hs) + " |")
    return "\n".join(out)


def to_markdown(res) -> str:
    out = []
    for reg in res["regimes"]:
        out += [f"**{reg['regime']}** ({reg['params']})", "",
                "| configuration | state error | output error | retention | reversal | coherence |",
                "|---|---:|---:|---:|---:|---:|"]
        for r in reg["library"]:
            out.append(f"| {r['config']} | {r['state_err']:.3e} | {r['out_err']:.3e} | {r['retention']:.3f} | "
                       f"{r['reversal']:.4f} | {r['coherence']:.3f} |")
        if reg["grouping"]:
            out += ["", "| qbits | rounding | value axis | key axis | per head |", "|---:|---|---:|---:|---:|"]
            for g in reg["grouping"]:
                out.append(f"| {g['qbits']} | {g['rounding']} | {g['value']:.3e} | {g['key']:.3e} | "
                           f"{g['head']:.3e} |")
        out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--B", type=int, default=16)
    ap.add_argument("--T", type=int, default=256)
    ap.add_argument("--json", default=None)
    ap.add_argument("--horizons", action="store_true", help="the decode-horizon table instead")
    args = ap.parse_args(argv)
    if args.horizons:
        res = [horizon_study(B=args.B, regime=reg) for reg in (REGIMES[2], REGIMES[-1])]
        print("\n\n".join(horizon_markdown(r) for r in res))
    else:
        res = study(B=args.B, T=args.T)
        print(to_markdown(res))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
