"""The pages' qualitative claims, reproduced through libqstate on synthetic
inputs with the structure they describe (a long context in the state,
persistent update directions, value channels of different magnitudes, slow
decay; see quantized_recurrent_state_qstate_amd.error_study):

* requantization with nearest rounding loses small updates and its errors
  are coherent from step to step, and stochastic rounding counters the
  accumulation ("Quantizing Recurrent Language Models Is Easier Than You
  Think", abstract; "Preserving Updates in Low-Bit Recurrent State
  Quantization", abstract);
* bounded directional rounding leaves no element moving against its update
  and lowers the error; the low-rank bypass lowers it further (the second
  page's abstract);
* scales grouped along the value axis beat key-axis and per-head scales (the
  first page's abstract).

The library's value-axis and key-axis nearest rounding also match an
independent float64 simulation of the same quantizer over the whole run."""
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_claims_reproduce_on_structured_inputs():
    from quantized_recurrent_state_qstate_amd import error_study as es
    rname, rp = es.REGIMES[-1]
    print(f"[study] {rname}", file=sys.stderr, flush=True)
    res = es.study(B=4, H=2, T=128, regimes=[(rname, rp)])
    reg = res["regimes"][0]
    lib = {r["config"]: r for r in reg["library"]}
    grp = {(g["qbits"], g["rounding"]): g for g in reg["grouping"]}
    print(es.to_markdown(res), file=sys.stderr, flush=True)
    rtn4, sr4, bdr4, lrb4 = (lib[n] for n in ("int4 nearest", "int4 SR16", "int4 nearest+BDR",
                                              "int4 nearest+BDR+LRB r8"))
    rtn8, sr8 = lib["int8 nearest"], lib["int8 SR16"]
    # nearest rounding: coherent errors, lost updates; stochastic: unbiased
    assert rtn4["coherence"] > 0.5 and abs(sr4["coherence"]) < 0.1
    assert rtn4["retention"] < 0.3 and abs(sr4["retention"] - 1.0) < 0.05
    assert sr8["state_err"] < 0.5 * rtn8["state_err"] and sr4["state_err"] < 0.6 * rtn4["state_err"]
    # directional rounding and the bypass
    assert bdr4["reversal"] < 1e-4 < rtn4["reversal"]
    assert bdr4["state_err"] < rtn4["state_err"]
    assert lrb4["state_err"] < bdr4["state_err"]
    # scale grouping
    g8 = grp[(8, "nearest")]
    assert g8["value"] < g8["key"] < g8["head"]
    # the library against a float64 simulation of the same quantizer, over the
    # whole run, for the row and the key-channel groups
    for axis in ("value", "key"):
        sim = es.run_grouping(axis, 8, "nearest", 4, 2, 128, 128, 128, rp, 2024)
        assert abs(g8[axis] - sim) <= 0.05 * sim, (axis, g8[axis], sim)


def test_low_precision_fares_best_on_short_horizons():
    """Errors accumulate with the decode horizon (i.i.d. updates, very slow
    decay, from an empty state): int4 with stochastic rounding (no buffer)
    after 64 steps is well below its own error after 1024, and int8's error
    stays below int4's at every horizon."""
    from quantized_recurrent_state_qstate_amd import error_study as es
    print("[study] horizons", file=sys.stderr, flush=True)
    res = es.horizon_study(B=4, H=2, horizons=(64, 256, 1024), regime=es.REGIMES[2])
    print(es.horizon_markdown(res), file=sys.stderr, flush=True)
    rows = {r["config"]: r["at"] for r in res["rows"]}
    sr4, sr8 = rows["int4 SR16"], rows["int8 SR16"]
    assert sr4[64]["state_err"] < 0.5 * sr4[1024]["state_err"]
    assert sr4[64]["state_err"] < sr4[256]["state_err"] < sr4[1024]["state_err"]
    for h in (64, 256, 1024):
        assert sr8[h]["state_err"] < sr4[h]["state_err"]
