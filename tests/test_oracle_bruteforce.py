"""Exhaustive and statistical pins of the oracle's rounding.

* Exhaustive 4x4 int4: every row of four int4 codes (15^4 = 50625 rows, as
  50625 one-row heads of width 4) takes one step; the oracle's new codes must
  equal a brute-force search over the 15 levels, done here in fp64 on the
  oracle's own pre-rounding values: the nearest level (ties to even) for
  nearest rounding, and for BDR ("round reversed elements toward their
  updates", page on preserving updates) the nearest level among those on the
  update's side of the old value.  fp64 and the oracle's fp32 x = S*(Q/max)
  may disagree only where x lies within 1e-5 of a decision boundary.
* Stochastic rounding across 2048 seeds: the mean rounding error of every
  element is zero within its standard error plus the 2^-17 LSB bias bound
  of 16-bit stochastic rounding (unbiasedness, LoReS abstract),
  and neighbouring elements' errors are uncorrelated (each element draws its
  own bits).
"""
import itertools

import numpy as np
import pytest

import oracle


def _all_rows():
    lv = np.arange(-7, 8)
    return np.array(list(itertools.product(lv, lv, lv, lv)), np.int32)   # [50625, 4]


def _pack_int4(codes):
    c = codes.astype(np.int32) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8).reshape(-1)


def _unpack_int4(b, n):
    b = b.reshape(n, -1)
    lo, hi = (b & 0xF).astype(np.int32), (b >> 4).astype(np.int32)
    out = np.empty((n, b.shape[1] * 2), np.int32)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out)


@pytest.mark.parametrize("bdr", [False, True])
def test_exhaustive_4x4_int4(bdr):
    rows = _all_rows()
    n = rows.shape[0]
    r = np.random.default_rng(17)
    cfg = oracle.Cfg(B=n, H=1, dk=4, dv=1, qbits=4, rounding="rtn", bdr=bdr, decay_mode="key")
    st = oracle.new_state(cfg)
    codes_b = _pack_int4(rows)
    # head blocks are padded to 16 bytes: row bytes = 2, block = 16
    st["codes"].reshape(n, 16)[:, :2] = codes_b.reshape(n, 2)
    scale = np.float32(0.1)
    st["scales"][:] = scale
    q = r.standard_normal((n, 1, 4)).astype(np.float32)
    k = (r.standard_normal((n, 1, 4)) * 0.05).astype(np.float32)
    v = r.standard_normal((n, 1, 1)).astype(np.float32)
    d = (1 / (1 + np.exp(-r.standard_normal((n, 1, 4)) - 3))).astype(np.float32)
    o, sp = oracle.step(cfg, st, q, k, v, d, None, step=0, want_sp=True)
    sp = sp.reshape(n, 4).astype(np.float64)
    # the pre-rounding value is the exact update of the dequantized codes
    ex = d.reshape(n, 4).astype(np.float64) * (scale * rows) + v.reshape(n, 1) * k.reshape(n, 4)
    np.testing.assert_allclose(sp, ex, rtol=0, atol=1e-6 * (np.abs(ex).max() + 1))
    new = _unpack_int4(st["codes"].reshape(n, 16)[:, :2].reshape(-1), n)
    m = np.abs(sp).max(1, keepdims=True)
    x = np.where(m > 0, sp * 7.0 / np.where(m > 0, m, 1), 0)
    xo = np.where(m > 0, (scale * rows) * 7.0 / np.where(m > 0, m, 1), 0)
    D = sp - scale * rows
    levels = np.arange(-7, 8, dtype=np.float64)
    dist = np.abs(x[..., None] - levels)                          # [n,4,15]
    if bdr:
        side_ok = (levels - xo[..., None]) * np.sign(D)[..., None] >= 0
        side_ok |= (D == 0)[..., None]
        dist = np.where(side_ok, dist, np.inf)
    best = dist.min(-1, keepdims=True)
    cand = np.isclose(dist, best, rtol=0, atol=1e-12)
    # ties to even: among equal-distance levels prefer the even one
    even = (np.abs(levels) % 2 == 0)
    pick = np.where(cand & even, 1, 0) + np.where(cand, 1, 0)
    bf = levels[pick.argmax(-1)]
    # no level on the update's side inside the grid: the clamp keeps the limit
    bf = np.where(np.isinf(best[..., 0]), np.clip(np.where(D > 0, np.ceil(x), np.floor(x)), -7, 7), bf)
    bad = new != bf
    frac = np.abs(x - np.floor(x) - 0.5)
    near_boundary = (frac < 1e-5) | (np.abs(x - np.round(x)) < 1e-5) | (np.abs(x - xo) < 1e-5)
    assert not (bad & ~near_boundary).any(), np.argwhere(bad & ~near_boundary)[:5]
    assert bad.sum() <= 50


def test_sr_unbiased_and_independent_over_seeds():
    r = np.random.default_rng(23)
    B, H, dv, dk = 1, 1, 4, 64
    S = r.standard_normal((B, H, dv, dk)).astype(np.float32)
    nseeds = 2048
    errs = np.empty((nseeds, dv, dk))
    for s in range(nseeds):
        cfg = oracle.Cfg(B=B, H=H, dk=dk, dv=dv, rounding="sr", seed=s * 7919 + 1)
        st = oracle.new_state(cfg)
        oracle.quantize(cfg, S, st, step=s)
        errs[s] = (oracle.dequantize(cfg, st) - S)[0, 0]
    lsb = (np.abs(S[0, 0]).max(-1) / 127.0)[:, None]
    mean = errs.mean(0) / lsb
    # each code is floor(x) or floor(x)+1 with probability p = frac(x): the
    # standard deviation of one error is sqrt(p (1 - p)) LSB
    x = S[0, 0].astype(np.float64) / lsb
    p = x - np.floor(x)
    sd = np.sqrt(p * (1 - p))
    # 256 elements: every mean error (in LSB) within 4.5 standard errors (two
    # sided 7e-6 each) plus the rounding's bias bound 2^-17 and fp32 slack
    assert (np.abs(mean) <= 4.5 * sd / np.sqrt(nseeds) + 2.0 ** -17 + 1e-6).all()
    assert np.abs(mean).max() < 0.05
    # neighbouring elements use different bits: correlation ~ 0
    e = errs / lsb
    a, b = e[:, :, :-1].reshape(nseeds, -1), e[:, :, 1:].reshape(nseeds, -1)
    a, b = a - a.mean(0), b - b.mean(0)
    corr = (a * b).mean(0) / (a.std(0) * b.std(0) + 1e-12)
    assert np.abs(corr.mean()) < 0.02
