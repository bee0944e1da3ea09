"""Decode steps captured in a HIP graph replay to the same state and outputs
as the same launches run eagerly.

A step enqueues only its kernel on the caller's stream (no allocation, copy or
memset), so a serving loop may capture a run of steps and replay it.  Each
case captures three steps, replays the graph three times with unrelated eager
work and synchronizations in between, and after every replay compares every
state buffer and output bit for bit with the same three steps run eagerly on
a second state.
"""
import sys

import numpy as np
import pytest
import torch

from quantized_recurrent_state_qstate_amd import QState, StateConfig

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "dense_headmap_bf16_sr": dict(kind="additive", decay_mode="head", dk=128, dv=64, H=4, B=3, qbits=8,
                                  map_mode="head", hp_dtype="bf16"),
    "dense_delta_4lanes": dict(kind="delta", decay_mode="head", dk=128, dv=128, H=2, B=2, qbits=8),
    "keymap_fp16_delta": dict(kind="delta", decay_mode="head", dk=128, dv=40, H=2, B=2, qbits=8,
                              map_mode="key", hp_dtype="fp16"),
    "lrb_int4_bdr_merges": dict(kind="additive", decay_mode="key", dk=128, dv=64, H=2, B=2, qbits=4,
                                rounding="nearest", bdr=True, lrb_rank=8, lrb_period=2),
    "grouped_key_axis": dict(kind="additive", decay_mode="key", dk=64, dv=40, H=3, B=2, qbits=8,
                             scale_axis="key"),
}

STEPS = [5, 6, 7]   # captured step indices (with period 2, steps 5 and 7 merge)


def _inputs(kw, seed):
    g = torch.Generator().manual_seed(seed)
    B, H, dk, dv = kw["B"], kw["H"], kw["dk"], kw["dv"]
    q = torch.randn(B, H, dk, generator=g) * 0.3
    k = torch.randn(B, H, dk, generator=g)
    k = k / k.norm(dim=-1, keepdim=True) if kw["kind"] == "delta" else k * 0.3
    v = torch.randn(B, H, dv, generator=g)
    shape = (B, H, dk) if kw["decay_mode"] == "key" else (B, H)
    d = torch.sigmoid(torch.randn(shape, generator=g) + 3)
    beta = torch.sigmoid(torch.randn(B, H, generator=g)) if kw["decay_mode"] == "head" or kw["kind"] == "delta" \
        else None
    dev = lambda x: None if x is None else x.to(DEV)
    return dict(q=dev(q.to(torch.bfloat16)), k=dev(k.to(torch.bfloat16)), v=dev(v.to(torch.bfloat16)),
                decay=dev(d), beta=dev(beta))


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(case):
    kw = dict(CASES[case])
    r = np.random.default_rng(2)
    m = None
    if kw.get("map_mode") == "head":
        m = (np.arange(kw["H"]) % 2).astype(np.uint8)
    elif kw.get("map_mode") == "key":
        m = (r.random((kw["H"], kw["dk"])) < 0.2).astype(np.uint8)
    kw.setdefault("rounding", "stochastic")
    qs = QState(StateConfig(map=m, seed=0x5EED, **kw))
    print(f"[graph] {case}: {qs.kernel_name}", file=sys.stderr, flush=True)
    st_g, st_e = qs.new_state(), qs.new_state()
    inp = [_inputs(kw, 100 + t) for t in range(len(STEPS))]
    for t in range(2):   # a state that is not all zeros, the same in both
        warm = _inputs(kw, 50 + t)
        qs.step(st_g, **warm, step=t)
        qs.step(st_e, **warm, step=t)
    out_g = [torch.empty(kw["B"], kw["H"], kw["dv"], device=DEV) for _ in STEPS]
    out_e = [torch.empty_like(o) for o in out_g]
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for t, s in enumerate(STEPS):
                qs.step(st_g, **inp[t], out=out_g[t], step=s)
    torch.cuda.synchronize()

    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.randn(1 << 18, device=DEV) * 2.0).sum().item()   # unrelated eager work
        for t, s in enumerate(STEPS):
            qs.step(st_e, **inp[t], out=out_e[t], step=s)
        torch.cuda.synchronize()
        for name in st_g:
            assert _same(st_g[name], st_e[name]), f"{case}: replay {rep}, state {name} differs"
        for t in range(len(STEPS)):
            assert _same(out_g[t], out_e[t]), f"{case}: replay {rep}, output of step {STEPS[t]} differs"
    qs.close()
