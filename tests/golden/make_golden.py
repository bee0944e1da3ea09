"""Writes the fixtures of this folder.  Run from the repository root:

    python tests/golden/make_golden.py

The pages (two abstracts) print no worked example, so two kinds of fixture
stand here:

* closed_form_*.json: a step whose result follows from the definitions by
  hand, written with plain numpy from those definitions (no oracle, no
  library): a zero state, one-hot keys and queries.  After the step, row v
  of a head holds v_v at key j and zeros elsewhere ("Quantizing Recurrent
  Language Models Is Easier Than You Think", abstract: the state matrix and
  its per-step update), so its scale is |v_v| / Q (value-axis grouping, the
  same abstract), its code at key j is sign(v_v) Q and every other code 0,
  and the readout is o_v = v_v.
* oracle_*.json: regression fixtures written by the oracle alone (this
  script calls oracle/ and numpy, nothing else): the initial fp32 state,
  the inputs of three steps, and the stored state and outputs after each.
  They fix the oracle's results, so a change to its arithmetic shows here
  and has to be made on purpose (regenerate with this script, naming the
  passage or reading that justifies it).

Arrays are stored as the hex of their little-endian bytes with dtype and
shape, so every value round-trips exactly.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def enc(a) -> dict:
    a = np.ascontiguousarray(a)
    return {"dtype": a.dtype.str, "shape": list(a.shape), "hex": a.tobytes().hex()}


def dec(d: dict) -> np.ndarray:
    return np.frombuffer(bytes.fromhex(d["hex"]), dtype=np.dtype(d["dtype"])).reshape(d["shape"]).copy()


def _write(name, obj):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(obj, f, indent=1)
        f.write("\n")


# ---------------------------------------------------------------------------
# Closed form
# ---------------------------------------------------------------------------
def closed_form(qbits: int) -> dict:
    B, H, dk, dv = 1, 2, 64, 24
    Q = 127 if qbits == 8 else 7
    r = np.random.default_rng(31 + qbits)
    v = (r.standard_normal((B, H, dv)) * 3).astype(np.float32)
    v[0, 0, 5] = 0.0                      # a zero row: scale 0, codes 0
    v[0, 1, 7] = -v[0, 1, 7]              # both signs in each head
    j = [3, 60]                           # the one-hot key (and query) of each head
    k = np.zeros((B, H, dk), np.float32)
    q = np.zeros((B, H, dk), np.float32)
    for h in range(H):
        k[0, h, j[h]] = 1.0
        q[0, h, j[h]] = 1.0
    decay = np.full((B, H), 0.5, np.float32)   # acts on a zero state
    # expected: codes, scales, readout from the definitions
    codes = np.zeros((B, H, dv, dk), np.int32)
    scales = np.zeros((B, H, dv), np.float32)
    for h in range(H):
        for row in range(dv):
            m = np.float32(abs(v[0, h, row]))
            if m > 0:
                scales[0, h, row] = m / np.float32(Q)            # IEEE fp32 quotient
                codes[0, h, row, j[h]] = Q if v[0, h, row] > 0 else -Q
    if qbits == 8:
        code_bytes = codes.astype(np.int8).view(np.uint8).reshape(-1)
    else:
        nib = (codes & 0xF).astype(np.uint8).reshape(B, H, dv, dk // 2, 2)
        code_bytes = (nib[..., 0] | (nib[..., 1] << 4)).reshape(-1)
    o = v.copy()
    return {
        "what": f"closed form, int{qbits} nearest: zero state, one-hot k = q = e_j per head, one step",
        "cite": "Quantizing Recurrent Language Models Is Easier Than You Think, abstract (state matrix "
                "updated per step; value-axis scale grouping)",
        "config": dict(kind="additive", decay_mode="head", B=B, H=H, dk=dk, dv=dv, qbits=qbits,
                       rounding="nearest", seed=0),
        "S0": None,
        "steps": [{"t": 0, "q": enc(q), "k": enc(k), "v": enc(v), "decay": enc(decay), "beta": None,
                   "o": enc(o), "state": {"codes": enc(code_bytes), "scales": enc(scales.reshape(-1))}}],
    }


# ---------------------------------------------------------------------------
# Oracle regression
# ---------------------------------------------------------------------------
ORACLE_CASES = {
    "oracle_gla_int8_sr16": dict(
        what="GLA-style additive step, per-key decay, int8 with 16-bit stochastic rounding",
        cite="Quantizing Recurrent Language Models Is Easier Than You Think, abstract (stochastic "
             "rounding); Salmon et al., SC'11, Philox section (Philox4x32-10)",
        config=dict(kind="additive", decay_mode="key", B=1, H=2, dk=64, dv=24, qbits=8,
                    rounding="stochastic", sr_bits=16, seed=0x5EED_0001)),
    "oracle_gdn_int8_sr8_headmap_bf16": dict(
        what="delta rule, per-head decay, int8 with 8-bit stochastic rounding, head 1 kept in bf16",
        cite="Quantizing Recurrent Language Models Is Easier Than You Think, abstract (decay-based mixed "
             "precision); Preserving Updates in Low-Bit Recurrent State Quantization, abstract (Gated DeltaNet)",
        config=dict(kind="delta", decay_mode="head", B=1, H=2, dk=64, dv=24, qbits=8,
                    rounding="stochastic", sr_bits=8, map_mode="head", hp_dtype="bf16", map=[0, 1],
                    seed=0x5EED_0002)),
    "oracle_gla_int4_bdr_lrb": dict(
        what="additive step, per-key decay, int4 nearest with BDR and a rank-4 low-rank bypass "
             "(merge period 2; keys 0..15 are small every step, so their updates are buffered and "
             "merged within the eight steps)",
        cite="Preserving Updates in Low-Bit Recurrent State Quantization, abstract (INT4, Low-Rank Bypass, "
             "Bounded Directional Rounding)",
        config=dict(kind="additive", decay_mode="key", B=1, H=2, dk=64, dv=24, qbits=4,
                    rounding="nearest", bdr=True, lrb_rank=4, lrb_period=2, lrb_theta=0.5, seed=0)),
}


def oracle_cfg(c: dict):
    import oracle
    kw = dict(c)
    kw["rounding"] = "rtn" if kw["rounding"] == "nearest" else "sr"
    if kw.get("map") is not None:
        kw["map"] = np.asarray(kw["map"], np.uint8)
    return oracle.Cfg(**kw)


def case_inputs(c: dict, t: int, seed: int):
    r = np.random.default_rng(seed * 1000 + t)
    B, H, dk, dv = c["B"], c["H"], c["dk"], c["dv"]
    q = (r.standard_normal((B, H, dk)) / 8).astype(np.float32)
    k = r.standard_normal((B, H, dk))
    if c.get("lrb_rank"):
        # keys 0..15 small and the same every step, v mostly one direction:
        # their updates fall below the buffer's threshold, build up in it
        # with one sign and reach the merge threshold within a few steps
        k[..., :16] = 0.02
    if c["kind"] == "delta":
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = r.standard_normal((B, H, dv))
    if c.get("lrb_rank"):
        v = 2.0 * np.random.default_rng(seed).standard_normal((B, H, dv)) + 0.1 * v
    v = v.astype(np.float32)
    shape = (B, H, dk) if c["decay_mode"] == "key" else (B, H)
    decay = (1 / (1 + np.exp(-(3 + r.standard_normal(shape))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32) if c["kind"] == "delta" else None
    return q, k, v, decay, beta


def oracle_case(name: str, spec: dict) -> dict:
    import oracle
    c = spec["config"]
    cfg = oracle_cfg(c)
    seed = sum(map(ord, name))
    r = np.random.default_rng(seed)
    S0 = (r.standard_normal((c["B"], c["H"], c["dv"], c["dk"])) * 0.5).astype(np.float32)
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, S0, st, step=0)
    out = {"what": spec["what"], "cite": spec["cite"], "config": c, "S0": enc(S0), "quantize_step": 0,
           "state0": {kk: enc(vv) for kk, vv in st.items()}, "steps": []}
    merges = 0
    for t in range(1, 9 if c.get("lrb_rank") else 4):
        q, k, v, decay, beta = case_inputs(c, t, seed)
        if c.get("lrb_rank"):
            o, _, _, merged, _, _ = oracle.step_lrb_trace(cfg, st, q, k, v, decay, beta, step=t)
            merges += int(merged.sum())
        else:
            o = oracle.step(cfg, st, q, k, v, decay, beta, step=t)
        out["steps"].append({"t": t, "q": enc(q), "k": enc(k), "v": enc(v), "decay": enc(decay),
                             "beta": None if beta is None else enc(beta), "o": enc(np.asarray(o, np.float32)),
                             "state": {kk: enc(vv) for kk, vv in st.items()}})
    if c.get("lrb_rank"):
        assert merges > 0, f"{name}: no channel merged"
        out["merged_channels"] = merges
    return out


def main():
    for qb in (8, 4):
        _write(f"closed_form_int{qb}.json", closed_form(qb))
    for name, spec in ORACLE_CASES.items():
        _write(f"{name}.json", oracle_case(name, spec))
    print("wrote", sorted(f for f in os.listdir(HERE) if f.endswith(".json")))


if __name__ == "__main__":
    main()
