"""Pins of the oracle's number formats, stochastic rounding and precision map.

* bf16 / fp16 storage of protected units (decay-based mixed precision, LoReS
  abstract) must be round-to-nearest-even: checked against torch's
  independent float -> bfloat16 / float16 conversions, over random values,
  exact ties, subnormals, overflow and signed zeros.
* stochastic rounding (LoReS abstract): enumerating all 2^16 (2^8) random
  integers gives the exact expectation: x rounded to 16 (8) fractional bits
  (halves up), within 2^-17 (2^-9) of x.
* the map builder keeps the round-half-up(frac * n) units of smallest decay
  rate per group, ties to the lower index (hand-made statistics).
* the row inverse Q / max rounded toward zero is the largest fp32 whose
  product with max does not exceed Q (exact rational arithmetic), so every
  element of the row scales into [-Q, Q] (and [-Q 2^b, Q 2^b] for
  stochastic rounding) without clamping.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _values():
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(4000).astype(np.float32) * s for s in (1e-3, 1.0, 1e3)]
    bits = rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32)
    vals.append(bits.view(np.float32))
    # exact ties for bf16 (low 16 bits = 0x8000) and fp16 (13 dropped bits = 0x1000)
    base = rng.integers(0x3F800000, 0x47000000, 500, dtype=np.uint64).astype(np.uint32)
    vals.append(((base & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32))
    vals.append(((base & ~np.uint32(0x1FFF)) | np.uint32(0x1000)).view(np.float32))
    sub = rng.integers(1, 0x00800000, 500, dtype=np.uint64).astype(np.uint32)
    vals.append(sub.view(np.float32))
    vals.append(np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, -65520.0, 3.4e38,
                          5.96e-8, 2.98e-8, 2.99e-8, 6.1e-5, 1e-45], np.float32))
    v = np.concatenate(vals)
    return v[np.isfinite(v) | np.isinf(v)]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_rne_16bit_matches_torch(fmt):
    v = _values()
    tdt = torch.bfloat16 if fmt == "bf16" else torch.float16
    ref = torch.from_numpy(v).to(tdt).view(torch.int16).numpy().astype(np.uint16)
    conv = oracle.to_bf16 if fmt == "bf16" else oracle.to_fp16
    got = np.array([conv(float(x)) for x in v], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_16bit_widening_matches_torch(fmt):
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    tdt = torch.bfloat16 if fmt == "bf16" else torch.float16
    ref = torch.from_numpy(bits.view(np.int16)).view(tdt).float().numpy()
    dec = oracle.from_bf16 if fmt == "bf16" else oracle.from_fp16
    got = np.array([dec(int(b)) for b in bits], np.float32)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("bits", [16, 8])
@pytest.mark.parametrize("x", [0.0, 3.0, -5.0, 0.3, -0.3, 2.75, -126.0001, 126.99, 1.0 / 3.0, 6.5e-5,
                               0.5 + 2.0 ** -17, -7.0 - 2.0 ** -9])
def test_sr_expectation_exact(bits, x):
    """Enumerating every random integer: outcomes are floor(x) or floor(x)+1 and
    their mean is x rounded to `bits` fractional bits (halves up)."""
    x = float(np.float32(x))
    n = 1 << bits
    xb = float(np.float32(x) * np.float32(n))          # exact scaling
    outs = np.array([oracle.sr_round(xb, u, bits) for u in range(n)])
    f = np.floor(x)
    assert set(np.unique(outs)) <= {f, f + 1}
    mean = outs.mean()
    assert mean == np.floor(x * n + 0.5) / n
    assert abs(mean - x) <= 2.0 ** -(bits + 1)
    if x == f:
        assert (outs == x).all()   # values on the grid never move


def test_map_builder_hand_cases():
    # one group of 8 heads: 25% -> 2 smallest rates
    stat = np.array([3.0, 0.5, 2.0, 0.1, 4.0, 0.5, 9.0, 1.0])
    assert oracle.build_map(stat, 1, 8, 0.25).tolist() == [0, 1, 0, 1, 0, 0, 0, 0]
    # ties go to the lower index
    stat = np.array([1.0, 0.2, 0.2, 0.2, 5.0])
    assert oracle.build_map(stat, 1, 5, 0.4).tolist() == [0, 1, 1, 0, 0]
    # all equal -> lowest indices; 10% of 128 = 12.8 -> 13
    m = oracle.build_map(np.full(2 * 128, 0.7), 2, 128, 0.10).reshape(2, 128)
    assert (m[:, :13] == 1).all() and (m[:, 13:] == 0).all()
    # half-up: 0.25 * 6 = 1.5 -> 2
    assert oracle.build_map(np.arange(6.0)[::-1].copy(), 1, 6, 0.25).tolist() == [0, 0, 0, 0, 1, 1]
    # frac 0 and 1
    assert oracle.build_map(np.arange(4.0), 1, 4, 0.0).sum() == 0
    assert oracle.build_map(np.arange(4.0), 1, 4, 1.0).sum() == 4


def _magnitudes():
    rng = np.random.default_rng(11)
    m = [rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 3000)]
    m.append(rng.integers(0x00800000, 0x7F000000, 3000, dtype=np.uint64).astype(np.uint32).view(np.float32))
    m.append(np.array([1.0, 127.0, 7.0, 0.5, 3.0, 1.0 / 3.0, 2.0 ** -100, 1e-30, 3.0e30], np.float32))
    m = np.abs(np.concatenate(m)).astype(np.float32)
    return m[(m > 0) & np.isfinite(m)]


@pytest.mark.parametrize("q", [127.0, 7.0])
def test_inverse_scale_rounds_toward_zero(q):
    for m in _magnitudes():
        m = float(m)
        if q / m * 65536.0 >= 2.0 ** 127:      # inverse (times 2^16) near fp32 overflow
            continue
        f = oracle.inv_rtz(q, m)
        assert Fraction(f) * Fraction(m) <= Fraction(q)
        up = float(np.nextafter(np.float32(f), np.float32(np.inf)))
        assert Fraction(up) * Fraction(m) > Fraction(q), (m, f)


@pytest.mark.parametrize("q", [127.0, 7.0])
def test_scaled_row_never_exceeds_q(q):
    rng = np.random.default_rng(12)
    for _ in range(300):
        row = (rng.standard_normal(64) * 10.0 ** rng.uniform(-20, 20)).astype(np.float32)
        m = float(np.abs(row).max())
        inv = np.float32(oracle.inv_rtz(q, m))
        for bits in (0, 8, 16):
            invb = np.float32(inv * np.float32(2.0 ** bits))      # exact scaling
            x = row * invb                                        # fp32 products, nearest
            assert np.abs(x).max() <= q * 2.0 ** bits
        assert np.abs(row * inv).max() >= q * (1 - 2.0 ** -22)  # the maximum reaches Q
