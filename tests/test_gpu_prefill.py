"""Prefill hand-off (the step before decode in a server): a state produced by
the test harness's chunked parallel prefill (float64, tests/prefill.py) goes
through qstate_quantize, then decodes through libqstate.

* quantize of the prefill state: codes, scales and protected values equal
  the oracle's quantize of the same fp32 state, bit for bit;
* the decode steps after it: teacher-forced against the oracle, to the usual
  parity bar;
* the decoded outputs follow the exact recurrence continued from the prefill
  state within a sound bound of the quantizer's error: each requantization
  adds less than one LSB of its row (half under nearest rounding, 2^-8 of the
  value for 16-bit protected heads), decayed by the later steps, seen
  through |q|."""
import sys

import numpy as np
import pytest
import torch

import oracle
from prefill import chunked_prefill, workload_sequence
from quantized_recurrent_state_qstate_amd import QState
from quantized_recurrent_state_qstate_amd.workloads import WORKLOADS

from helpers import gpu_state_to_oracle, inputs_f32, lib_cfg, oracle_cfg
from test_gpu_parity import compare

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name", ["mamba2", "gla_int4_sr", "gla_small"])
def test_prefill_state_hands_off_to_decode(name):
    w = WORKLOADS[name]
    B, T0, N = 2, 48, 6
    print(f"[prefill] {name} B={B} prefill {T0} decode {N}", file=sys.stderr, flush=True)
    q, k, u, a = workload_sequence(w, B, T0 + N)
    S, _ = chunked_prefill(np.zeros((B, w.H, w.dv, w.dk)), q[:T0], k[:T0], u[:T0], a[:T0], C=16)
    S32 = np.ascontiguousarray(S, dtype=np.float32)
    ocfg = oracle_cfg(w, B=B)
    qs = QState(lib_cfg(w, B=B))
    st = qs.new_state()
    qs.quantize(torch.from_numpy(S32).to(DEV), st, step=T0)
    torch.cuda.synchronize()
    ost = oracle.new_state(ocfg)
    oracle.quantize(ocfg, S32, ost, step=T0)
    got = gpu_state_to_oracle(st, w.hp_dtype)
    assert np.array_equal(got["codes"], ost["codes"])
    assert np.array_equal(got["scales"], ost["scales"])
    assert np.array_equal(got["hp"].view(np.uint8), ost["hp"].view(np.uint8))
    # sound elementwise bound of the decode's error against the exact
    # continuation: every requantization adds less than one LSB of its row
    # (half under nearest rounding; 2^-8 of the value for 16-bit protected
    # units), and earlier errors decay with the state
    lsb = 0.5 if w.rounding == "nearest" else 1.0
    prot = np.zeros((w.H,), bool)
    if w.map_mode == "head":
        prot = np.asarray(ocfg.map, bool)

    def new_error(st_np, S_exact):
        sc = oracle.widen(st_np["scales"]).reshape(B, w.H, w.dv)[..., None] * lsb
        return np.where(prot[None, :, None, None], 2.0 ** -8 * np.abs(S_exact), np.broadcast_to(sc, S_exact.shape))

    S_ex = S
    E = new_error(got, S_ex)
    worst = 0.0
    for t in range(T0, T0 + N):
        inp = w.step_inputs(t, B)
        ref = gpu_state_to_oracle(st, w.hp_dtype)
        o_ref = oracle.step(ocfg, ref, **inputs_f32(inp), step=t)
        o = qs.step(st, **{n: (None if x is None else x.to(DEV)) for n, x in inp.items()}, step=t)
        torch.cuda.synchronize()
        og = o.cpu().numpy().astype(np.float64)
        now = gpu_state_to_oracle(st, w.hp_dtype)
        compare(ocfg, w.kind == "additive" and not w.lrb_rank, ref, now, o_ref, o.cpu().numpy(),
                what=f"{name} after prefill t={t}")
        S_ex = S_ex * a[t][..., None, :] + u[t][..., :, None] * k[t][..., None, :]
        o_ex = np.einsum("...vk,...k->...v", S_ex, q[t])
        E = E * a[t][..., None, :]                      # earlier errors, decayed; the output sees these
        slack = 1e-5 * np.einsum("...vk,...k->...v", np.abs(S_ex), np.abs(q[t])) + 1e-30
        bound = np.einsum("...vk,...k->...v", E, np.abs(q[t])) + slack
        err = np.abs(og - o_ex)
        assert (err <= bound).all(), f"{name} t={t}: output error {(err / bound).max():.2f} x its bound"
        worst = max(worst, float((err / bound).max()))
        E = E + new_error(now, S_ex)                    # this step's requantization
    print(f"[prefill] {name}: largest output error / its bound {worst:.3f}", file=sys.stderr)
    qs.close()
