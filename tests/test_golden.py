"""The fixtures of tests/golden against the oracle (CPU).

* closed_form_int{8,4}: the oracle, from a zero state, takes the one step
  whose codes, scales and readout follow from the definitions by hand
  (see tests/golden/make_golden.py) and must give exactly those values;
* oracle_*: the oracle replays the stored inputs from the stored initial
  fp32 state and must give the stored states and outputs bit for bit, so a
  change to its arithmetic fails here until the fixtures are rewritten on
  purpose.  Each fixture is also checked to exercise what it names.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def dec(d):
    return np.frombuffer(bytes.fromhex(d["hex"]), dtype=np.dtype(d["dtype"])).reshape(d["shape"]).copy()


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def ocfg(c):
    kw = dict(c)
    kw["rounding"] = "rtn" if kw["rounding"] == "nearest" else "sr"
    if kw.get("map") is not None:
        kw["map"] = np.asarray(kw["map"], np.uint8)
    return oracle.Cfg(**kw)


def step_args(s):
    return dict(q=dec(s["q"]), k=dec(s["k"]), v=dec(s["v"]), decay=dec(s["decay"]),
                beta=None if s["beta"] is None else dec(s["beta"]))


def test_fixtures_present_and_cited():
    names = sorted(os.path.basename(p) for p in glob.glob(os.path.join(GOLDEN, "*.json")))
    assert {"closed_form_int8.json", "closed_form_int4.json"} <= set(names)
    assert sum(n.startswith("oracle_") for n in names) >= 3
    for n in names:
        fx = load(n)
        assert fx["cite"] and fx["what"], n


@pytest.mark.parametrize("qbits", [8, 4])
def test_closed_form(qbits):
    fx = load(f"closed_form_int{qbits}.json")
    cfg = ocfg(fx["config"])
    st = oracle.new_state(cfg)
    s = fx["steps"][0]
    o = oracle.step(cfg, st, **step_args(s), step=s["t"])
    assert np.array_equal(st["codes"], dec(s["state"]["codes"]))
    assert np.array_equal(st["scales"].view(np.uint32), dec(s["state"]["scales"]).view(np.uint32))
    assert np.array_equal(np.asarray(o, np.float32).reshape(-1), dec(s["o"]).reshape(-1))


ORACLE_FIXTURES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(GOLDEN, "oracle_*.json")))


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("name", ORACLE_FIXTURES)
def test_oracle_regression(name):
    fx = load(name)
    cfg = ocfg(fx["config"])
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, dec(fx["S0"]), st, step=fx["quantize_step"])
    for key, want in fx["state0"].items():
        assert np.array_equal(_bits(st[key]), _bits(dec(want))), f"{name} quantize: {key}"
    for s in fx["steps"]:
        o = oracle.step(cfg, st, **step_args(s), step=s["t"])
        assert np.array_equal(_bits(np.asarray(o, np.float32).reshape(-1)), _bits(dec(s["o"]).reshape(-1))), \
            f"{name} t={s['t']}: outputs"
        for key, want in s["state"].items():
            assert np.array_equal(_bits(st[key]), _bits(dec(want))), f"{name} t={s['t']}: {key}"


def test_oracle_fixtures_exercise_their_features():
    lrb = load("oracle_gla_int4_bdr_lrb.json")
    n = [dec(s["state"]["n"]) for s in lrb["steps"]]
    U = [dec(s["state"]["U"]) for s in lrb["steps"]]
    assert max(int(x.max()) for x in n) > 0                      # the basis grew
    assert any(np.any(u != 0) for u in U)                         # small updates were buffered
    assert lrb["merged_channels"] > 0                             # and some merged (oracle trace)
    cfg = ocfg(lrb["config"])
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, dec(lrb["S0"]), st, step=lrb["quantize_step"])
    merged = 0
    for s in lrb["steps"]:
        _, _, _, m, _, _ = oracle.step_lrb_trace(cfg, st, **step_args(s), step=s["t"])
        merged += int(m.sum())
    assert merged == lrb["merged_channels"]
    hm = load("oracle_gdn_int8_sr8_headmap_bf16.json")
    assert np.any(dec(hm["steps"][-1]["state"]["hp"]) != 0)       # the protected head is stored
    assert hm["config"]["kind"] == "delta" and hm["config"]["map"] == [0, 1]
    sr = load("oracle_gla_int8_sr16.json")
    assert sr["config"]["rounding"] == "stochastic" and sr["config"]["sr_bits"] == 16
