"""Pins of the oracle's scale grouping axes.

The LoReS abstract ("Quantizing Recurrent Language Models Is Easier Than You
Think") groups scales along the value axis to match output channel magnitude.
The oracle also takes the groupings that reading is chosen over, as an
ablation: one scale per key channel (a column of S[v][k]) and one per head.

Pinned against other code paths of the oracle and against the recurrence:
* key axis on S equals value axis on S^T (codes and scales), for quantize and
  for one additive step with a per-head decay, under nearest rounding (the
  transposed problem swaps the roles of u and k; fma is symmetric in them);
* one scale per head equals the value axis of the head flattened into one
  row, for quantize under both roundings (the element indices coincide);
* one step under each axis equals the exact recurrence plus a rounding error
  of at most half an LSB of the element's group (nearest), with the group's
  scale its largest magnitude over Q bitwise and the largest element of each
  group at code +-Q; both kinds, both decay modes.
"""
import numpy as np
import pytest

import oracle
from oracle import fp64


def _codes_and_scales(cfg, st):
    """Codes [B,H,dv,dk] read from the stored rows (every channel quantized)
    and scales [B,H,G]."""
    L = oracle.layout(cfg)
    rb = ((cfg.dk * cfg.qbits + 7) // 8 + 3) // 4 * 4
    codes = np.zeros((cfg.B, cfg.H, cfg.dv, cfg.dk))
    for b in range(cfg.B):
        for h in range(cfg.H):
            base = b * L["code_bstride"] + int(L["code_off"][h])
            for v in range(cfg.dv):
                row = st["codes"][base + v * rb: base + (v + 1) * rb]
                if cfg.qbits == 8:
                    codes[b, h, v] = row[:cfg.dk].view(np.int8)
                else:
                    nib = np.stack([row & 0xF, row >> 4], 1).reshape(-1)[:cfg.dk].astype(np.int64)
                    codes[b, h, v] = np.where(nib >= 8, nib - 16, nib)
    G = {"value": cfg.dv, "key": cfg.dk, "head": 1}[cfg.scale_axis]
    return codes, st["scales"].reshape(cfg.B, cfg.H, G).astype(np.float64)


def _state(r, B, H, dv, dk):
    return (r.standard_normal((B, H, dv, dk)) * np.exp(r.uniform(-2, 2, (B, H, dv, 1)))
            * np.exp(r.uniform(-2, 2, (B, H, 1, dk)))).astype(np.float32)


@pytest.mark.parametrize("qbits", [8, 4])
def test_key_axis_is_value_axis_of_the_transpose(qbits):
    r = np.random.default_rng(qbits)
    B, H, dv, dk = 2, 2, 12, 20
    S = _state(r, B, H, dv, dk)
    ck = oracle.Cfg(B=B, H=H, dk=dk, dv=dv, qbits=qbits, rounding="rtn", scale_axis="key")
    cv = oracle.Cfg(B=B, H=H, dk=dv, dv=dk, qbits=qbits, rounding="rtn", scale_axis="value")
    sk, sv = oracle.new_state(ck), oracle.new_state(cv)
    oracle.quantize(ck, S, sk)
    oracle.quantize(cv, np.ascontiguousarray(S.transpose(0, 1, 3, 2)), sv)
    codes_k, s_k = _codes_and_scales(ck, sk)
    codes_v, s_v = _codes_and_scales(cv, sv)
    assert np.array_equal(s_k, s_v)
    assert np.array_equal(codes_k, codes_v.transpose(0, 1, 3, 2))


@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_head_axis_is_value_axis_of_the_flattened_head(rounding):
    r = np.random.default_rng(5)
    B, H, dv, dk = 2, 3, 6, 16
    S = _state(r, B, H, dv, dk)
    ch = oracle.Cfg(B=B, H=H, dk=dk, dv=dv, qbits=4, rounding=rounding, scale_axis="head", seed=11)
    cf = oracle.Cfg(B=B, H=H, dk=dv * dk, dv=1, qbits=4, rounding=rounding, scale_axis="value", seed=11)
    sh, sf = oracle.new_state(ch), oracle.new_state(cf)
    oracle.quantize(ch, S, sh, step=4)
    oracle.quantize(cf, S.reshape(B, H, 1, dv * dk), sf, step=4)
    assert np.array_equal(sh["codes"], sf["codes"])
    assert np.array_equal(sh["scales"], sf["scales"])


def test_key_axis_step_is_value_axis_step_of_the_transpose():
    """Additive step, one decay per head: S_pre = d S + u k^T.  Transposed,
    S^T_pre = d S^T + k u^T, the same recurrence with u' = k (beta' = 1) and
    k' = u; element by element fma(u_v, k_k, (d s_k) c) = fma(k_k, u_v, ...)."""
    r = np.random.default_rng(9)
    B, H, dv, dk = 2, 2, 12, 20
    ck = oracle.Cfg(B=B, H=H, dk=dk, dv=dv, qbits=8, rounding="rtn", scale_axis="key", decay_mode="head")
    cv = oracle.Cfg(B=B, H=H, dk=dv, dv=dk, qbits=8, rounding="rtn", scale_axis="value", decay_mode="head")
    sk, sv = oracle.new_state(ck), oracle.new_state(cv)
    S = _state(r, B, H, dv, dk)
    oracle.quantize(ck, S, sk)
    oracle.quantize(cv, np.ascontiguousarray(S.transpose(0, 1, 3, 2)), sv)
    for t in range(6):
        q = r.standard_normal((B, H, dk)).astype(np.float32)
        k = r.standard_normal((B, H, dk)).astype(np.float32)
        v = r.standard_normal((B, H, dv)).astype(np.float32)
        beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32)
        d = (1 / (1 + np.exp(-r.standard_normal((B, H)) - 3))).astype(np.float32)
        u = (beta[..., None] * v).astype(np.float32)            # u = beta v in fp32, as the step forms it
        oracle.step(ck, sk, q, k, v, d, beta, step=t)
        oracle.step(cv, sv, np.ones((B, H, dv), np.float32), u, k, d, None, step=t)
        codes_k, s_k = _codes_and_scales(ck, sk)
        codes_v, s_v = _codes_and_scales(cv, sv)
        assert np.array_equal(s_k, s_v), t
        assert np.array_equal(codes_k, codes_v.transpose(0, 1, 3, 2)), t


@pytest.mark.parametrize("axis", ["key", "head", "value"])
@pytest.mark.parametrize("kind,decay_mode", [("additive", "key"), ("additive", "head"), ("delta", "head"),
                                             ("delta", "key")])
@pytest.mark.parametrize("qbits", [8, 4])
def test_step_is_exact_recurrence_plus_half_lsb_of_the_group(axis, kind, decay_mode, qbits):
    r = np.random.default_rng(3)
    B, H, dv, dk = 2, 2, 12, 16
    Q = 127 if qbits == 8 else 7
    cfg = oracle.Cfg(kind=kind, decay_mode=decay_mode, B=B, H=H, dk=dk, dv=dv, qbits=qbits, rounding="rtn",
                     scale_axis=axis)
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, _state(r, B, H, dv, dk), st)
    for t in range(4):
        S_prev = oracle.dequantize(cfg, st).astype(np.float64)
        q = r.standard_normal((B, H, dk)).astype(np.float32)
        k = r.standard_normal((B, H, dk))
        if kind == "delta":
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        k = k.astype(np.float32)
        v = r.standard_normal((B, H, dv)).astype(np.float32)
        shape = (B, H, dk) if decay_mode == "key" else (B, H)
        d = (1 / (1 + np.exp(-r.standard_normal(shape) - 3))).astype(np.float32)
        beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32)
        _, sp = oracle.step(cfg, st, q, k, v, d, beta, step=t, want_sp=True)
        ex = (fp64.delta_step(S_prev, q, k, v, d, beta) if kind == "delta"
              else fp64.additive_step(S_prev, q, k, v, d, beta))[0]
        codes, s = _codes_and_scales(cfg, st)
        sp = sp.astype(np.float64)
        # the group scale is the group's largest |S_pre| over Q, bitwise
        if axis == "value":
            m, se = np.abs(sp).max(-1), s[..., :, None]
        elif axis == "key":
            m, se = np.abs(sp).max(-2), s[..., None, :]
        else:
            m, se = np.abs(sp).max((-1, -2))[..., None], s[..., None]
        assert np.array_equal(s.astype(np.float32), (m.astype(np.float32) / np.float32(Q)).astype(np.float32))
        D = se * codes
        assert (np.abs(D - sp) <= 0.5 * se * (1 + 2.0 ** -20)).all()
        assert (np.abs(sp - ex) <= 1e-5 * (np.abs(ex).max() + 1)).all()      # S_pre is the exact step
        # the largest element of each group lands on +-Q
        top = np.abs(codes)
        top = top.max(-1) if axis == "value" else (top.max(-2) if axis == "key" else top.max((-1, -2))[..., None])
        assert (top[m > 0] == Q).all()
