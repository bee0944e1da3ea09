"""Pins of the oracle's bf16 storage layout: bf16 row scales and bf16 factors
of the low-rank buffer.

The page on preserving updates reports that INT4 states with the Low-Rank
Bypass reduce state memory by up to 5.3x against FP32 states.  At a 128 x 128
head that figure is reached with int4 codes plus a rank-8 buffer whose two
factors are 16-bit: 64 KiB / (8 KiB + 2 x 2 KiB) = 5.33.  The oracle's reading
of that layout:

* a row's scale is stored as bf16, rounded up: the smallest bf16 value s with
  Q s >= m (m the row's largest magnitude), and codes are taken against the
  stored scale, x = value * inv with inv the largest float not above 1 / s,
  so |x| <= Q and no code needs clamping;
* W and U are stored as bf16 (nearest even).  A new basis column is rounded
  when it is made and used rounded in that step; U is updated in fp32 from
  its stored values and rounded before the merge test, so the merge, the
  readout and the stored state see the same buffer.

Pinned here against independent constructions: the rounded-up scale against
a search over all positive bf16 values in exact rational arithmetic; the
rounding bounds of codes taken against a bf16 scale; the buffer's bookkeeping
up to its own rounding (the effective state after a step is one exact step of
the one before, off by no more than half a bf16 unit of each stored U entry
times |W|); the readout against the stored buffer; W near-orthonormal.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import fp64

# every positive finite bf16 value, ascending with its bit pattern
_BF16_POS = np.arange(1, 0x7F80, dtype=np.uint32)
_BF16_VAL = (_BF16_POS << 16).view(np.float32)


def _scale_up_reference(m, q):
    """Smallest bf16 value s with q s >= m, by bisection over the ascending
    bf16 values with exact rational comparisons."""
    target = Fraction(float(m)) / q
    lo, hi = 0, _BF16_VAL.size - 1
    if Fraction(float(_BF16_VAL[hi])) < target:
        return float("inf")
    while lo < hi:
        mid = (lo + hi) // 2
        if Fraction(float(_BF16_VAL[mid])) >= target:
            hi = mid
        else:
            lo = mid + 1
    return float(_BF16_VAL[lo])


@pytest.mark.parametrize("q", [127, 7])
def test_scale_rounded_up_to_bf16(q):
    r = np.random.default_rng(q)
    bits = r.integers(0x00000001, 0x7F800000, 3000, dtype=np.uint64).astype(np.uint32)
    ms = list(bits.view(np.float32))
    # edges: exact bf16 multiples of q, bf16 values themselves, just above/below them, the top
    for b in (0x3F80, 0x3E12, 0x0080, 0x0001, 0x7F7F):
        v = float((np.uint32(b) << 16).view(np.float32))
        if v * q >= 3.4e38:
            ms.append(np.float32(v))
            continue
        vq = np.float32(v * q)
        for m in (vq, np.nextafter(vq, np.float32(0)), np.nextafter(vq, np.float32(np.inf)), np.float32(v)):
            ms.append(np.float32(m))
    for m in ms:
        got = oracle.scale_bf16_up(float(m), float(q))
        want = _scale_up_reference(m, q)
        assert got == want, (float(m), q, got, want)


@pytest.mark.parametrize("qbits", [8, 4])
@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_codes_against_bf16_scale_within_bounds(qbits, rounding):
    Q = 127 if qbits == 8 else 7
    cfg = oracle.Cfg(B=2, H=2, dk=64, dv=16, qbits=qbits, rounding=rounding, scale_dtype="bf16", seed=4)
    r = np.random.default_rng(qbits)
    S = (r.standard_normal((2, 2, 16, 64)) * np.exp(r.uniform(-30, 30, (2, 2, 16, 1)))).astype(np.float32)
    S[0, 0, 0] = 0.0
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, S, st, step=1)
    s = oracle.widen(st["scales"]).reshape(2, 2, 16)
    D = oracle.dequantize(cfg, st).astype(np.float64)
    codes = np.where(s[..., None] > 0, D / np.where(s[..., None] > 0, s[..., None], 1), 0)
    assert np.array_equal(codes, np.round(codes)) and np.abs(codes).max() <= Q
    m = np.abs(S.astype(np.float64)).max(-1)
    for idx in np.ndindex(m.shape):
        if m[idx] == 0:
            assert s[idx] == 0 and not codes[idx].any()
            continue
        assert s[idx] == _scale_up_reference(np.float32(m[idx]), Q)
    err = np.abs(D - S)
    lim = (0.5 if rounding == "rtn" else 1.0) * s[..., None] * (1 + 2.0 ** -20)
    assert (err <= lim).all()
    if rounding == "rtn":
        # the largest element lands within one code of Q (s exceeds m/Q by less than a bf16 unit)
        top = np.abs(codes).max(-1)
        assert (top[m > 0] >= Q - 1).all()


def _cfg(kind, decay_mode, scale_dtype):
    return oracle.Cfg(kind=kind, decay_mode=decay_mode, B=2, H=2, dk=16, dv=12, qbits=4, rounding="rtn", bdr=True,
                      lrb_rank=3, lrb_period=4, lrb_theta=0.5, seed=9, scale_dtype=scale_dtype, lrb_dtype="bf16")


def _inputs(cfg, r):
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = r.standard_normal((B, H, dk)).astype(np.float32)
    k = r.standard_normal((B, H, dk))
    if cfg.kind == "delta":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k[..., dk // 2:] *= 0.05
    k = k.astype(np.float32)
    v = r.standard_normal((B, H, dv)).astype(np.float32)
    shape = (B, H, dk) if cfg.decay_mode == "key" else (B, H)
    d = (1 / (1 + np.exp(-r.standard_normal(shape) - 4))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32) if cfg.kind == "delta" else None
    return q, k, v, d, beta


def _factors(cfg, st):
    r = cfg.lrb_rank
    W = oracle.widen(st["W"]).reshape(cfg.B * cfg.H, cfg.dv, r)
    U = oracle.widen(st["U"]).reshape(cfg.B * cfg.H, cfg.dk, r)
    return W, U


@pytest.mark.parametrize("kind", ["additive", "delta"])
@pytest.mark.parametrize("decay_mode", ["key", "head"])
@pytest.mark.parametrize("scale_dtype", ["fp32", "bf16"])
def test_bf16_buffer_bookkeeping_up_to_its_rounding(kind, decay_mode, scale_dtype):
    cfg = _cfg(kind, decay_mode, scale_dtype)
    r = np.random.default_rng(7)
    st = oracle.new_state(cfg)
    BH, dv, dk = cfg.B * cfg.H, cfg.dv, cfg.dk
    merges = grown = 0
    for t in range(24):
        S_prev = oracle.dequantize(cfg, st).astype(np.float64)
        n_before = st["n"].copy()
        _, U_before = _factors(cfg, st)
        q, k, v, d, beta = _inputs(cfg, r)
        o, sp = oracle.step(cfg, st, q, k, v, d, beta, step=t, want_sp=True)
        W, U = _factors(cfg, st)
        L = np.stack([W[i, :, :st["n"][i]] @ U[i, :, :st["n"][i]].T for i in range(BH)]).reshape(
            cfg.B, cfg.H, dv, dk)
        eff = sp.astype(np.float64) + L
        ex = (fp64.delta_step(S_prev, q, k, v, d, beta) if kind == "delta"
              else fp64.additive_step(S_prev, q, k, v, d))[0]
        # half a bf16 unit (2^-8 relative) of every U entry as it was rounded,
        # through |W|: a merged channel was rounded before it was cleared, so
        # its entries are bounded by the decayed entry before the step plus
        # the step's addition |k_k| |c| <= |k_k| |u|
        if kind == "delta":
            dd = d[..., None, :] if decay_mode == "key" else d[..., None, None]
            u = beta[..., None] * (v - np.einsum("bhvk,bhk->bhv", S_prev * dd, k.astype(np.float64)))
        else:
            u = v.astype(np.float64)
        un = np.linalg.norm(u, axis=-1).reshape(BH) * 1.01
        Ub = np.abs(U_before) + (np.abs(k.reshape(BH, dk)) * un[:, None])[..., None]
        absWU = np.stack([np.abs(W[i]) @ np.maximum(np.abs(U[i]), Ub[i]).T for i in range(BH)]).reshape(
            cfg.B, cfg.H, dv, dk)
        tol = 2.0 ** -8 * absWU + 2e-6 * (np.abs(ex).max() + 1)
        assert (np.abs(eff - ex) <= tol).all(), (t, (np.abs(eff - ex) / tol).max())
        # the readout sees exactly the stored buffer
        o_stored = np.einsum("bhvk,bhk->bhv", eff, q.astype(np.float64))
        np.testing.assert_allclose(o, o_stored, rtol=0, atol=2e-6 * (np.abs(eff).max() + 1) * np.abs(q).sum(-1).max())
        grown += int((st["n"] > n_before).sum())
        merges += int((t + 1) % cfg.lrb_period == 0)
    assert grown > 0 and merges > 0
    W, U = _factors(cfg, st)
    assert np.abs(U).max() > 0
    for i in range(BH):
        n = st["n"][i]
        G = W[i, :, :n].T @ W[i, :, :n]
        assert np.abs(G - np.eye(n)).max() <= 2.0 ** -7


def test_bf16_layout_state_bytes_at_the_pages_shape():
    """128 x 128 heads, int4 codes, rank-8 bf16 factors, bf16 scales: the
    state is 5.22x smaller than fp32 (5.33x without the scales)."""
    cfg = oracle.Cfg(B=1, H=1, dk=128, dv=128, qbits=4, rounding="rtn", bdr=True, lrb_rank=8,
                     scale_dtype="bf16", lrb_dtype="bf16")
    L = oracle.layout(cfg)
    state = L["codes"] + L["scales"] + L["W"] + L["U"] + L["n"]
    assert (L["codes"], L["scales"], L["W"], L["U"]) == (8192, 256, 2048, 2048)
    fp32 = 128 * 128 * 4
    assert abs(fp32 / state - 5.22) < 0.01
    assert abs(fp32 / (L["codes"] + L["W"] + L["U"]) - 5.333) < 0.001


# Planted mistakes in copies of the oracle's source (CPU only): each must
# fail the pins above.
MUTANTS = {
    # the scale rounded to nearest instead of up (codes may then exceed Q)
    "scale_nearest": ("    g.scale = orc_scale_bf16_up(m, Q);\n",
                      "    g.scale = orc_from_bf16(orc_to_bf16(m / Q));\n"),
    # a new basis column used unrounded in its first step (stored rounded)
    "basis_unrounded": ("W[v * r + n] = lrb_round(c, y[v] / ny);", "W[v * r + n] = y[v] / ny;"),
    # the buffer rounded only when stored, after the merge test and readout
    "buffer_rounded_late": ("  for (int i = 0; i < dk * r; ++i) U[i] = lrb_round(c, U[i]);\n", ""),
}


def _mutant_library(tmp, name):
    import os
    import shutil
    import subprocess
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "qs_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site of {name} not found once in the oracle"
    cpath = os.path.join(tmp, f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src.replace(old, new))
    shutil.copy(os.path.join(here, "qs_oracle.h"), tmp)
    so = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-I", tmp, cpath, "-o", so, "-lm"], check=True, capture_output=True)
    return so


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name):
    import tempfile
    pins = [lambda: test_codes_against_bf16_scale_within_bounds(8, "rtn"),
            lambda: test_codes_against_bf16_scale_within_bounds(4, "sr")]
    pins += [(lambda a=a, b=b, c=c: test_bf16_buffer_bookkeeping_up_to_its_rounding(a, b, c))
             for a in ("additive", "delta") for b in ("key", "head") for c in ("fp32", "bf16")]
    failed = 0
    with tempfile.TemporaryDirectory() as tmp:
        with oracle.using(_mutant_library(tmp, name)):
            for pin in pins:
                try:
                    pin()
                except AssertionError:
                    failed += 1
    assert failed > 0, f"no pin caught the planted mistake {name}"
