"""Pins of the oracle over whole runs: how rounding errors accumulate under
repeated requantization (abstract of "Preserving Updates in Low-Bit Recurrent
State Quantization": the state is requantized after every update, so errors
accumulate; abstract of "Quantizing Recurrent Language Models Is Easier Than
You Think": stochastic rounding against that accumulation).

Additive recurrence with a decay per key channel (GLA), S[v][k]:
    exact:      S_t = S_{t-1} diag(d_t) + u_t k_t^T
    quantized:  S^q_t = S^q_{t-1} diag(d_t) + u_t k_t^T + E_t,
E_t the rounding residual of step t (plus fp32 rounding of the update).  The
difference D_t = S^q_t - S_t obeys D_t = D_{t-1} diag(d_t) + E_t, so
    D_T[v][k] = sum_t E_t[v][k] prod_{tau > t} d_tau[k].
* Nearest rounding: |E_t[v][k]| <= s_t[v] / 2 (s_t the row scale after step
  t), so |D_T[v][k]| <= sum_t (s_t[v] / 2) prod_{tau>t} d_tau[k], plus the
  fp32 slack.  A floor in place of nearest (errors up to 1 LSB, all one way)
  or a decay applied twice breaks the bound.
* Stochastic rounding: E_t has mean within 2^-17 s_t of zero (16 random bits)
  and variance at most s_t^2 / 4 given the past, so over seeds D_T has mean
  about 0 and variance at most sum_t (s_t^2 / 4) prod_{tau>t} d_tau^2.
"""
import numpy as np
import pytest

import oracle
from oracle import fp64

B, H, DK, DV = 1, 2, 16, 12


def _inputs(r, T):
    qs = r.standard_normal((T, B, H, DK)).astype(np.float32)
    ks = (0.5 * r.standard_normal((T, B, H, DK))).astype(np.float32)
    vs = r.standard_normal((T, B, H, DV)).astype(np.float32)
    ds = (1 / (1 + np.exp(-(r.standard_normal((T, B, H, DK)) + 3)))).astype(np.float32)
    return qs, ks, vs, ds


def _run(cfg, S0, inputs, seed_steps=0):
    """Quantized run from quantize(S0); returns the dequantized start, the
    dequantized end state, and the scales after every step [T,B,H,DV]."""
    qs, ks, vs, ds = inputs
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, S0, st, step=seed_steps)
    start = oracle.dequantize(cfg, st).astype(np.float64)
    scales = []
    for t in range(len(qs)):
        oracle.step(cfg, st, qs[t], ks[t], vs[t], ds[t], step=seed_steps + 1 + t)
        scales.append(st["scales"].reshape(B, H, DV).astype(np.float64).copy())
    return start, oracle.dequantize(cfg, st).astype(np.float64), np.array(scales)


def _decay_after(ds):
    """prod_{tau > t} d_tau[k] for every t: [T,B,H,DK] (float64)."""
    d = ds.astype(np.float64)
    out = np.ones_like(d)
    for t in range(len(d) - 2, -1, -1):
        out[t] = out[t + 1] * d[t + 1]
    return out


@pytest.mark.parametrize("qbits", [8, 4])
def test_nearest_rounding_error_within_accumulated_half_lsb(qbits):
    T = 64
    r = np.random.default_rng(11 + qbits)
    cfg = oracle.Cfg(kind="additive", decay_mode="key", B=B, H=H, dk=DK, dv=DV, qbits=qbits, rounding="rtn")
    inputs = _inputs(r, T)
    S0 = (2 * r.standard_normal((B, H, DV, DK))).astype(np.float32)
    start, end, scales = _run(cfg, S0, inputs)
    states, _ = fp64.run("additive", start, *inputs)
    err = np.abs(end - states[-1])                                       # [B,H,DV,DK]
    P = _decay_after(inputs[3])                                          # [T,B,H,DK]
    half = 0.5 * scales[..., :, None] * P[..., None, :]                  # [T,B,H,DV,DK]
    mag = np.abs(np.array(states))                                       # fp32 slack of each update
    bound = half.sum(0) + (2.0 ** -21 * mag * P[..., None, :]).sum(0)
    assert (err <= bound).all(), (err / bound).max()
    # the bound is not vacuous: the error reaches a fair share of it somewhere
    assert (err / bound).max() > 0.2


def test_nearest_bound_catches_one_sided_rounding():
    """The same bound fails for a run whose every rounding goes down (floor):
    errors up to 1 LSB, all of one sign, accumulate past the half-LSB sum."""
    T = 64
    r = np.random.default_rng(5)
    inputs = _inputs(r, T)
    qs, ks, vs, ds = inputs
    S = (2 * r.standard_normal((B, H, DV, DK))).astype(np.float64)
    exact = S.copy()
    Q = 127.0
    half = np.zeros_like(S)
    P = _decay_after(ds)
    for t in range(T):
        exact, _ = fp64.additive_step(exact, qs[t], ks[t], vs[t], ds[t])
        S, _ = fp64.additive_step(S, qs[t], ks[t], vs[t], ds[t])
        s = np.abs(S).max(-1, keepdims=True) / Q
        S = np.floor(S / s) * s                                           # one-sided rounding
        half += 0.5 * s * P[t][..., None, :]
    assert (np.abs(S - exact) > half).any()


@pytest.mark.parametrize("qbits", [8, 4])
def test_stochastic_rounding_unbiased_over_seeds_with_bounded_variance(qbits):
    T, N = 32, 400
    r = np.random.default_rng(21 + qbits)
    inputs = _inputs(r, T)
    S0 = (2 * r.standard_normal((B, H, DV, DK))).astype(np.float32)
    P2 = _decay_after(inputs[3]) ** 2
    D, V, bias = [], np.zeros((B, H, DV, DK)), np.zeros((B, H, DV, DK))
    for seed in range(N):
        cfg = oracle.Cfg(kind="additive", decay_mode="key", B=B, H=H, dk=DK, dv=DV, qbits=qbits, rounding="sr",
                         sr_bits=16, seed=1000 + seed)
        start, end, scales = _run(cfg, S0, inputs)
        states, _ = fp64.run("additive", start, *inputs)
        D.append(end - states[-1])
        V += ((scales ** 2 / 4)[..., :, None] * P2[..., None, :]).sum(0)
        bias += ((2.0 ** -17 * scales + 2.0 ** -21 * np.abs(np.array(states)).max(-1))[..., :, None]
                 * np.sqrt(P2)[..., None, :]).sum(0)
    D = np.array(D)
    V /= N
    bias /= N
    mean = D.mean(0)
    # mean within 5 standard errors (plus the bounded bias) in every element
    assert (np.abs(mean) <= 5 * np.sqrt(V / N) + bias).all(), (np.abs(mean) / np.sqrt(V / N)).max()
    # variance within the bound (sampling noise of a variance over 400 seeds: ~7%)
    assert (D.var(0) <= 1.3 * V).all(), (D.var(0) / V).max()
    # and the errors are real: the variance is a fair share of the bound
    assert (D.var(0) / V).mean() > 0.3
