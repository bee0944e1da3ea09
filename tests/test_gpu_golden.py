"""The fixtures of tests/golden against the HIP library, through the C ABI.

* closed form: from a zero state, one step must give the hand-derived codes,
  scales and readout exactly;
* oracle fixtures: quantize of the stored fp32 state must give the stored
  state bit for bit; then each step, started from the stored state before it
  (teacher-forced), must match the stored state and outputs to the parity
  bar of the live oracle comparisons (exact for additive steps without the
  buffer, the documented tolerances otherwise).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from quantized_recurrent_state_qstate_amd import QState, StateConfig

from helpers import gpu_state_to_oracle, oracle_state_to_gpu
from test_golden import GOLDEN, ORACLE_FIXTURES, dec, load, ocfg
from test_gpu_parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


def lcfg(c):
    kw = dict(c)
    if kw.get("map") is not None:
        kw["map"] = np.asarray(kw["map"], np.uint8)
    return StateConfig(in_dtype="fp32", **kw)


def dev_args(s):
    out = {n: torch.from_numpy(dec(s[n])).to(DEV) for n in ("q", "k", "v", "decay")}
    out["beta"] = None if s["beta"] is None else torch.from_numpy(dec(s["beta"])).to(DEV)
    return out


@pytest.mark.parametrize("qbits", [8, 4])
def test_closed_form_on_gpu(qbits):
    fx = load(f"closed_form_int{qbits}.json")
    print(f"[golden] closed form int{qbits}", file=sys.stderr, flush=True)
    qs = QState(lcfg(fx["config"]))
    st = qs.new_state()
    s = fx["steps"][0]
    o = qs.step(st, **dev_args(s), step=s["t"])
    torch.cuda.synchronize()
    got = gpu_state_to_oracle(st, "bf16")
    assert np.array_equal(got["codes"], dec(s["state"]["codes"]))
    assert np.array_equal(got["scales"].view(np.uint32), dec(s["state"]["scales"]).view(np.uint32))
    assert np.array_equal(o.cpu().numpy().reshape(-1), dec(s["o"]).reshape(-1))
    qs.close()


@pytest.mark.parametrize("name", ORACLE_FIXTURES)
def test_oracle_fixture_on_gpu(name):
    fx = load(name)
    c = fx["config"]
    print(f"[golden] {name}", file=sys.stderr, flush=True)
    oc = ocfg(c)
    qs = QState(lcfg(c))
    st = qs.new_state()
    qs.quantize(torch.from_numpy(dec(fx["S0"])).to(DEV), st, step=fx["quantize_step"])
    torch.cuda.synchronize()
    got = gpu_state_to_oracle(st, oc.hp_dtype)
    for key, want in fx["state0"].items():
        w = dec(want)
        g = got[key]
        assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), f"{name} quantize: {key}"
    exact = c["kind"] == "additive" and not c.get("lrb_rank")
    prev = {kk: dec(vv) for kk, vv in fx["state0"].items()}
    for s in fx["steps"]:
        st = oracle_state_to_gpu(prev, DEV)
        o = qs.step(st, **dev_args(s), step=s["t"])
        torch.cuda.synchronize()
        want = {kk: dec(vv) for kk, vv in s["state"].items()}
        compare(oc, exact, want, gpu_state_to_oracle(st, oc.hp_dtype), dec(s["o"]), o.cpu().numpy(),
                what=f"{name} t={s['t']}")
        prev = want
    qs.close()
