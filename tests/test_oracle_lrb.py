"""Pins of the oracle's Low-Rank Bypass (abstract of the page on preserving
updates: small updates accumulate in a compact low-rank buffer whose
sufficiently large elements are periodically merged into the state).

The reading implemented: buffer L = W U^T (W orthonormal value basis, U key
coefficients), decayed with the state, fed with the in-span part of the
update on key channels whose update is under theta LSB in every row, and on
merge steps channels reaching theta LSB are moved into the state.

* Exactness of the bookkeeping: the effective pre-rounding state (S_pre plus
  the buffer after the step) equals one exact fp64 step (additive, or delta
  rule on the effective state) of the previous effective state (dequantized
  codes plus buffer), and the output is that state times q -- across growth,
  accumulation and merge steps.  Any dropped decay, double-counted
  projection, delta pre-term that misses the buffer or merge that does not
  clear what it adds breaks this.
* A merge moves mass without changing the readout.
* After a merge every retained buffer channel is below theta LSB in every row.
* W has orthonormal columns.
* With no small channel (theta ~ 0) the codes equal those of the same run
  without the buffer.
"""
import numpy as np
import pytest

import oracle
from oracle import fp64


def _cfg(decay_mode="key", period=4, theta=0.5, rank=3, B=2, H=2, dk=16, dv=12, bdr=True, qbits=4,
         kind="additive"):
    return oracle.Cfg(kind=kind, B=B, H=H, dk=dk, dv=dv, qbits=qbits, rounding="rtn", bdr=bdr,
                      decay_mode=decay_mode, lrb_rank=rank, lrb_period=period, lrb_theta=theta, seed=9)


def _inputs(cfg, r, small_scale=0.05):
    """q, k, v, decay, beta.  The delta rule gets a unit-norm k whose second
    half is scaled down, and beta in (0, 1); additive kinds beta = None."""
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = r.standard_normal((B, H, dk)).astype(np.float32)
    k = r.standard_normal((B, H, dk))
    if cfg.kind == "delta":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k[..., dk // 2:] *= small_scale            # half the key channels carry small updates
    k = k.astype(np.float32)
    v = r.standard_normal((B, H, dv)).astype(np.float32)
    shape = (B, H, dk) if cfg.decay_mode == "key" else (B, H)
    d = (1 / (1 + np.exp(-r.standard_normal(shape) - 4))).astype(np.float32)
    beta = None
    if cfg.kind == "delta":
        beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32)
    return q, k, v, d, beta


def _exact_step(cfg, S, q, k, v, d, beta):
    if cfg.kind == "delta":
        return fp64.delta_step(S, q, k, v, d, beta)
    return fp64.additive_step(S, q, k, v, d)


def _buffer(cfg, st):
    """L = W U^T of every head, via the oracle's dequantize with codes cleared."""
    z = {n: a.copy() for n, a in st.items()}
    z["codes"][:] = 0
    z["scales"][:] = 0
    return oracle.dequantize(cfg, z).astype(np.float64)


@pytest.mark.parametrize("kind", ["additive", "delta"])
@pytest.mark.parametrize("decay_mode", ["key", "head"])
@pytest.mark.parametrize("qbits", [4, 8])
def test_lrb_effective_state_is_exact(kind, decay_mode, qbits):
    """For the delta rule this also pins that the pre-term S k reads the
    buffer: dropping its W (U^T k) part leaves the state off by beta (L k) k^T."""
    cfg = _cfg(decay_mode=decay_mode, qbits=qbits, kind=kind)
    r = np.random.default_rng(3)
    st = oracle.new_state(cfg)
    merges = grown = 0
    for t in range(24):
        S_prev = oracle.dequantize(cfg, st).astype(np.float64)
        n_before = st["n"].copy()
        q, k, v, d, beta = _inputs(cfg, r)
        o, sp = oracle.step(cfg, st, q, k, v, d, beta, step=t, want_sp=True)
        L = _buffer(cfg, st)
        eff = sp.astype(np.float64) + L
        ex, o_ex = _exact_step(cfg, S_prev, q, k, v, d, beta)
        tol = 2e-6 * (np.abs(ex).max() + 1)
        np.testing.assert_allclose(eff, ex, rtol=0, atol=tol)
        np.testing.assert_allclose(o, o_ex, rtol=0, atol=tol * np.abs(q).sum(-1).max())
        grown += int((st["n"] > n_before).sum())
        if (t + 1) % cfg.lrb_period == 0:
            merges += 1
    assert grown > 0 and merges > 0
    # the buffer actually holds mass at the end of a non-merge stretch
    assert np.abs(_buffer(cfg, st)).max() > 0


@pytest.mark.parametrize("kind", ["additive", "delta"])
def test_merge_keeps_readout_and_clears_large_channels(kind):
    T = 16 if kind == "additive" else 32    # the delta rule's unit-norm keys fill the buffer slower
    cfg_m = _cfg(period=T, theta=0.5, kind=kind)
    cfg_n = _cfg(period=10 ** 9, theta=0.5, kind=kind)
    r = np.random.default_rng(8)
    st = oracle.new_state(cfg_n)
    for t in range(T - 1):
        q, k, v, d, beta = _inputs(cfg_n, r, small_scale=0.3)
        oracle.step(cfg_n, st, q, k, v, d, beta, step=t)
    st_n = {n: a.copy() for n, a in st.items()}
    s_old = st["scales"].reshape(cfg_m.B, cfg_m.H, cfg_m.dv).copy()
    q, k, v, d, beta = _inputs(cfg_m, r, small_scale=0.3)
    o_m = oracle.step(cfg_m, st, q, k, v, d, beta, step=T - 1)    # T % period == 0: merge
    o_n = oracle.step(cfg_n, st_n, q, k, v, d, beta, step=T - 1)  # same step, no merge
    np.testing.assert_allclose(o_m, o_n, rtol=0, atol=2e-6 * np.abs(o_n).max())
    L_m, L_n = _buffer(cfg_m, st), _buffer(cfg_n, st_n)
    merged = (np.abs(L_n).max(2) > 0) & (np.abs(L_m).max(2) == 0)
    assert merged.any(), "no channel reached the merge threshold"
    assert (np.abs(L_m).max(2) > 0).any(), "every channel merged"
    # every channel still in the buffer is below theta LSB in every row
    lsb = s_old[..., None].astype(np.float64)
    kept = np.abs(L_m).max(2) > 0                                  # [B,H,dk]
    ratio = np.where(lsb > 0, np.abs(L_m) / np.where(lsb > 0, lsb, 1), np.inf)
    assert not (kept[:, :, None, :] & (ratio >= cfg_m.lrb_theta)).any()


@pytest.mark.parametrize("kind", ["additive", "delta"])
def test_basis_is_orthonormal(kind):
    cfg = _cfg(rank=6, period=1000, kind=kind)
    r = np.random.default_rng(4)
    st = oracle.new_state(cfg)
    for t in range(10):
        q, k, v, d, beta = _inputs(cfg, r)
        oracle.step(cfg, st, q, k, v, d, beta, step=t)
    W = st["W"].reshape(cfg.B * cfg.H, cfg.dv, cfg.lrb_rank).astype(np.float64)
    for bh in range(cfg.B * cfg.H):
        n = st["n"][bh]
        assert n == cfg.lrb_rank
        G = W[bh, :, :n].T @ W[bh, :, :n]
        np.testing.assert_allclose(G, np.eye(n), atol=1e-5)


@pytest.mark.parametrize("kind", ["additive", "delta"])
def test_no_small_channel_equals_plain_run(kind):
    r1, r2 = np.random.default_rng(6), np.random.default_rng(6)
    cfg_l = _cfg(theta=1e-30, period=3, kind=kind)
    cfg_p = oracle.Cfg(kind=kind, B=cfg_l.B, H=cfg_l.H, dk=cfg_l.dk, dv=cfg_l.dv, qbits=4, rounding="rtn",
                       bdr=True, decay_mode="key", seed=9)
    st_l, st_p = oracle.new_state(cfg_l), oracle.new_state(cfg_p)
    for t in range(9):
        a = _inputs(cfg_l, r1)
        b = _inputs(cfg_p, r2)
        oracle.step(cfg_l, st_l, *a, step=t)
        oracle.step(cfg_p, st_p, *b, step=t)
    assert np.array_equal(st_l["codes"], st_p["codes"])
    assert np.array_equal(st_l["scales"], st_p["scales"])
    assert not st_l["U"].any()
