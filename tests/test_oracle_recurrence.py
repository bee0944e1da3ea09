"""Pins of the oracle's recurrences and of its quantized decode step.

1. The fp64 recurrences (oracle/fp64.py) against closed forms written
   differently: GLA as a sum of decayed rank-1 terms, Mamba2 as its
   quadratic (attention-like) form with the decay accumulated in the
   exponent, Gated DeltaNet as a product of transition matrices, plus special
   cases (beta = 0; alpha = beta = 1 with a unit key).
2. The quantized step (qs_oracle.c) against the pinned fp64 step: starting
   from the oracle's own dequantized state, its pre-rounding state S_pre and
   output o must equal one exact step of the recurrence to fp32 accuracy
   ("requantized after every update": the only error a step adds is its
   rounding), for every kind, decay mode, precision map and rounding.
3. Requantization: value-axis scale = max|S_pre| / Q over quantized channels
   (bitwise), codes in [-Q, Q], per-element error <= 0.5 LSB (nearest) or
   < 1 LSB (stochastic, BDR), protected channels = RNE bf16/fp16 of S_pre
   (torch's conversion), argmax element at |code| = Q under nearest rounding.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp64


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# 1. fp64 recurrences vs closed forms
# ---------------------------------------------------------------------------
def test_gla_closed_form():
    r = _rng(1)
    T, dv, dk = 9, 5, 6
    q, k = r.standard_normal((T, dk)), r.standard_normal((T, dk))
    v = r.standard_normal((T, dv))
    a = 1 / (1 + np.exp(-r.standard_normal((T, dk)) - 2))
    states, outs = fp64.run("additive", np.zeros((dv, dk)), q, k, v, a)
    for t in range(T):
        S = np.zeros((dv, dk))
        for s in range(t + 1):
            prod = np.ones(dk)
            for tau in range(s + 1, t + 1):
                prod = prod * a[tau]
            S += np.outer(v[s], k[s] * prod)
        np.testing.assert_allclose(states[t], S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(outs[t], S @ q[t], rtol=1e-12, atol=1e-12)


def test_mamba2_quadratic_form():
    r = _rng(2)
    T, P, N = 12, 4, 6
    x = r.standard_normal((T, P))
    Bm, Cm = r.standard_normal((T, N)), r.standard_normal((T, N))
    dt = np.log1p(np.exp(r.standard_normal(T) * 0.5 - 2))
    A = -np.exp(r.uniform(0, 2))
    _, outs = fp64.run("additive", np.zeros((P, N)), Cm, Bm, x, np.exp(dt * A), betas=dt)
    for t in range(T):
        y = np.zeros(P)
        for s in range(t + 1):
            y += (Cm[t] @ Bm[s]) * np.exp(A * dt[s + 1:t + 1].sum()) * dt[s] * x[s]
        np.testing.assert_allclose(outs[t], y, rtol=1e-10, atol=1e-12)


def test_gated_deltanet_transition_product():
    r = _rng(3)
    T, dv, dk = 8, 5, 7
    q, v = r.standard_normal((T, dk)), r.standard_normal((T, dv))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    al = 1 / (1 + np.exp(-r.standard_normal(T) - 3))
    be = 1 / (1 + np.exp(-r.standard_normal(T)))
    S0 = r.standard_normal((dv, dk))
    states, outs = fp64.run("delta", S0, q, k, v, al, betas=be)
    M = [al[t] * (np.eye(dk) - be[t] * np.outer(k[t], k[t])) for t in range(T)]
    for t in range(T):
        S = S0.copy()
        for tau in range(t + 1):
            S = S @ M[tau]
        for s in range(t + 1):
            term = be[s] * np.outer(v[s], k[s])
            for tau in range(s + 1, t + 1):
                term = term @ M[tau]
            S = S + term
        np.testing.assert_allclose(states[t], S, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(outs[t], S @ q[t], rtol=1e-11, atol=1e-12)


def test_channel_gated_delta_transition_product():
    """Delta rule with a decay per key channel: S_t = S_{t-1} M_t + beta_t v_t k_t^T
    with M_t = diag(d_t) (I - beta_t k_t k_t^T), checked against the dense product."""
    r = _rng(13)
    T, dv, dk = 7, 4, 6
    q, v = r.standard_normal((T, dk)), r.standard_normal((T, dv))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    d = 1 / (1 + np.exp(-r.standard_normal((T, dk)) - 2))
    be = 1 / (1 + np.exp(-r.standard_normal(T)))
    S0 = r.standard_normal((dv, dk))
    states, outs = fp64.run("delta", S0, q, k, v, d, betas=be)
    M = [np.diag(d[t]) @ (np.eye(dk) - be[t] * np.outer(k[t], k[t])) for t in range(T)]
    for t in range(T):
        S = S0.copy()
        for tau in range(t + 1):
            S = S @ M[tau]
        for s in range(t + 1):
            term = be[s] * np.outer(v[s], k[s])
            for tau in range(s + 1, t + 1):
                term = term @ M[tau]
            S = S + term
        np.testing.assert_allclose(states[t], S, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(outs[t], S @ q[t], rtol=1e-11, atol=1e-12)
    # equal channel decays reduce to the scalar-decay delta rule
    Sa, oa = fp64.delta_step(S0, q[0], k[0], v[0], np.full(dk, 0.7), be[0])
    Sb, ob = fp64.delta_step(S0, q[0], k[0], v[0], 0.7, be[0])
    np.testing.assert_allclose(Sa, Sb, rtol=1e-13, atol=1e-14)


def test_delta_special_cases():
    r = _rng(4)
    dv, dk = 4, 6
    S0 = r.standard_normal((dv, dk))
    q, v, k = r.standard_normal(dk), r.standard_normal(dv), r.standard_normal(dk)
    S, _ = fp64.delta_step(S0, q, k, v, 0.8, 0.0)          # beta = 0: pure decay
    np.testing.assert_allclose(S, 0.8 * S0, rtol=1e-15)
    e2 = np.eye(dk)[2]
    S, _ = fp64.delta_step(S0, q, e2, v, 1.0, 1.0)          # unit key: column 2 := v
    np.testing.assert_allclose(S[:, 2], v, rtol=1e-15)
    np.testing.assert_allclose(np.delete(S, 2, axis=1), np.delete(S0, 2, axis=1), rtol=1e-15)


# ---------------------------------------------------------------------------
# 2./3. quantized step vs the exact step of its own dequantized state
# ---------------------------------------------------------------------------
CASES = {
    "gla_int8_sr": dict(kind="additive", decay_mode="key", rounding="sr"),
    "gla_int8_rtn": dict(kind="additive", decay_mode="key", rounding="rtn"),
    "gla_int4_rtn_bdr": dict(kind="additive", decay_mode="key", rounding="rtn", qbits=4, bdr=True),
    "mamba2_headmap_sr": dict(kind="additive", decay_mode="head", rounding="sr", map_mode="head",
                              hp_dtype="bf16"),
    "gdn_sr": dict(kind="delta", decay_mode="head", rounding="sr"),
    "gdn_keymap_fp16_sr8": dict(kind="delta", decay_mode="head", rounding="sr", sr_bits=8,
                                map_mode="key", hp_dtype="fp16"),
    "gdn_int4_keymap_bdr": dict(kind="delta", decay_mode="head", rounding="sr", qbits=4, bdr=True,
                                map_mode="key", hp_dtype="bf16"),
    "kda_sr": dict(kind="delta", decay_mode="key", rounding="sr"),
    "kda_keymap_fp16_rtn": dict(kind="delta", decay_mode="key", rounding="rtn", map_mode="key",
                                hp_dtype="fp16"),
}


def _make(case, B=2, H=3, dk=16, dv=12, seed=11):
    kw = dict(CASES[case])
    r = _rng(seed)
    m = None
    if kw.get("map_mode") == "head":
        m = np.array([0, 1, 0], np.uint8)[:H]
    elif kw.get("map_mode") == "key":
        m = (r.random((H, dk)) < 0.25).astype(np.uint8)
        m[1, :] = 0   # one head fully quantized
        m[2, :] = 1   # one head fully protected
    cfg = oracle.Cfg(B=B, H=H, dk=dk, dv=dv, map=m, seed=1234, **kw)
    return cfg, r


def _inputs(cfg, r, t):
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = r.standard_normal((B, H, dk)).astype(np.float32)
    k = r.standard_normal((B, H, dk)).astype(np.float32)
    v = r.standard_normal((B, H, dv)).astype(np.float32)
    if cfg.kind == "delta":
        k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
        shape = (B, H, dk) if cfg.decay_mode == "key" else (B, H)
        d = (1 / (1 + np.exp(-r.standard_normal(shape) - 3))).astype(np.float32)
        beta = (1 / (1 + np.exp(-r.standard_normal((B, H))))).astype(np.float32)
    else:
        shape = (B, H, dk) if cfg.decay_mode == "key" else (B, H)
        d = (1 / (1 + np.exp(-r.standard_normal(shape) - 3))).astype(np.float32)
        beta = (r.random((B, H)) * 0.2).astype(np.float32) if cfg.decay_mode == "head" else None
    return q, k, v, d, beta


def _protected(cfg):
    H, dk = cfg.H, cfg.dk
    if cfg.map_mode == "none":
        return np.zeros((H, dk), bool)
    if cfg.map_mode == "head":
        return np.repeat(np.asarray(cfg.map, bool)[:, None], dk, axis=1)
    return np.asarray(cfg.map, bool).reshape(H, dk)


def _exact_step(cfg, S, q, k, v, d, beta):
    if cfg.kind == "delta":
        return fp64.delta_step(S, q, k, v, d, beta)
    return fp64.additive_step(S, q, k, v, d, beta)


@pytest.mark.parametrize("case", list(CASES))
def test_step_is_exact_recurrence_plus_rounding(case):
    cfg, r = _make(case)
    Q = 127 if cfg.qbits == 8 else 7
    st = oracle.new_state(cfg)
    prot = _protected(cfg)                       # [H, dk]
    for t in range(12):
        S_prev = oracle.dequantize(cfg, st).astype(np.float64)
        q, k, v, d, beta = _inputs(cfg, r, t)
        o, sp = oracle.step(cfg, st, q, k, v, d, beta, step=t, want_sp=True)
        S_ex, o_ex = _exact_step(cfg, S_prev, q, k, v, d, beta)
        scale_ref = np.abs(S_ex).max() + 1e-30
        np.testing.assert_allclose(sp, S_ex, rtol=0, atol=4e-7 * scale_ref)
        np.testing.assert_allclose(o, o_ex, rtol=0, atol=4e-7 * scale_ref * np.abs(q).sum(-1).max())

        # requantization pins
        S_new = oracle.dequantize(cfg, st)
        scales = st["scales"].reshape(cfg.B, cfg.H, cfg.dv)
        qmask = ~prot[None, :, None, :]          # [1,H,1,dk]
        absq = np.where(qmask, np.abs(sp), 0.0).max(-1)
        expect_scale = (absq.astype(np.float32) / np.float32(Q)).astype(np.float32)
        has_q = qmask.any(-1)
        assert np.array_equal(np.where(has_q, scales, 0), np.where(has_q, expect_scale, 0))
        err = np.abs(S_new.astype(np.float64) - sp)
        lsb = np.broadcast_to(scales[..., None], sp.shape).astype(np.float64)
        bound = (0.5 if (cfg.rounding == "rtn" and not cfg.bdr) else 1.0) * lsb * (1 + 2 ** -20)
        qm = np.broadcast_to(qmask, sp.shape)
        assert (err[qm] <= bound[qm] + 1e-30).all()
        codes = np.rint(np.where(lsb > 0, S_new / np.where(lsb > 0, lsb, 1), 0))
        assert (np.abs(codes[qm]) <= Q).all()
        if cfg.rounding == "rtn" and not cfg.bdr:
            # the row maximum sits at |code| == Q
            arg = np.where(qmask, np.abs(sp), -1).argmax(-1)
            top = np.take_along_axis(np.abs(codes), arg[..., None], -1)[..., 0]
            assert np.all((top == Q) | (scales == 0))
        # protected channels: RNE 16-bit of S_pre
        if prot.any():
            pm = np.broadcast_to(~qmask, sp.shape)
            tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[cfg.hp_dtype]
            ref = torch.from_numpy(sp).to(tdt).float().numpy()
            assert np.array_equal(S_new[pm], ref[pm])


def test_step_zero_inputs_keep_zero_state():
    cfg, r = _make("gla_int8_sr")
    st = oracle.new_state(cfg)
    z = np.zeros((cfg.B, cfg.H, cfg.dk), np.float32)
    o = oracle.step(cfg, st, z, z, np.zeros((cfg.B, cfg.H, cfg.dv), np.float32),
                    np.ones((cfg.B, cfg.H, cfg.dk), np.float32), None, step=0)
    assert not o.any() and not st["codes"].any() and not st["scales"].any()


def test_heads_subset_equals_full_run():
    cfg, r = _make("gdn_keymap_fp16_sr8")
    st_a = oracle.new_state(cfg)
    for t in range(3):
        q, k, v, d, beta = _inputs(cfg, r, t)
        oracle.step(cfg, st_a, q, k, v, d, beta, step=t)
    st_b = {n: a.copy() for n, a in st_a.items()}
    q, k, v, d, beta = _inputs(cfg, r, 3)
    o_a = oracle.step(cfg, st_a, q, k, v, d, beta, step=3)
    heads = np.array([4, 1], np.int64)
    o_b = oracle.step(cfg, st_b, q, k, v, d, beta, step=3, heads=heads)
    oa, ob = o_a.reshape(-1, cfg.dv), o_b.reshape(-1, cfg.dv)
    assert np.array_equal(oa[heads], ob[heads])
    Sa, Sb = oracle.dequantize(cfg, st_a), oracle.dequantize(cfg, st_b)
    Sa, Sb = Sa.reshape(-1, cfg.dv, cfg.dk), Sb.reshape(-1, cfg.dv, cfg.dk)
    assert np.array_equal(Sa[heads], Sb[heads])


@pytest.mark.parametrize("rounding", ["rtn", "sr"])
@pytest.mark.parametrize("qbits", [8, 4])
def test_quantize_roundtrip(rounding, qbits):
    r = _rng(5)
    cfg = oracle.Cfg(B=2, H=2, dk=16, dv=8, qbits=qbits, rounding=rounding, seed=3)
    Q = 127 if qbits == 8 else 7
    S = r.standard_normal((2, 2, 8, 16)).astype(np.float32)
    S[0, 1, 3] = 0.0                                  # a zero row
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, S, st, step=5)
    S2 = oracle.dequantize(cfg, st)
    lsb = (np.abs(S).max(-1, keepdims=True) / np.float32(Q)).astype(np.float32)
    assert np.array_equal(st["scales"].reshape(2, 2, 8), lsb[..., 0])
    k = 0.5 if rounding == "rtn" else 1.0
    assert (np.abs(S2 - S) <= k * lsb * (1 + 2 ** -20)).all()
    assert not S2[0, 1, 3].any()
    # values on the grid come back exactly
    on_grid = (S2 / np.where(lsb > 0, lsb, 1)).round() * lsb
    st2 = oracle.new_state(cfg)
    oracle.quantize(cfg, on_grid.astype(np.float32), st2, step=9)
    np.testing.assert_allclose(oracle.dequantize(cfg, st2), on_grid, rtol=2e-7, atol=0)


def test_layout_sizes_of_the_workloads():
    """Byte sizes of the documented layout, computed by hand for each workload."""
    def sizes(**kw):
        return oracle.layout(oracle.Cfg(**kw))
    z = sizes(B=1, H=2, dk=64, dv=64)
    assert (z["codes"], z["scales"], z["hp"]) == (2 * 64 * 64, 2 * 64 * 4, 0)
    z = sizes(B=64, H=32, dk=128, dv=128, kind="delta")
    assert (z["codes"], z["scales"]) == (64 * 32 * 128 * 128, 64 * 32 * 128 * 4)
    m = np.zeros(32, np.uint8)
    m[:8] = 1
    z = sizes(B=256, H=32, dk=128, dv=64, map_mode="head", map=m, hp_dtype="bf16")
    assert (z["codes"], z["hp"]) == (256 * 24 * 64 * 128, 256 * 8 * 64 * 128 * 2)
    z = sizes(B=128, H=32, dk=128, dv=128, qbits=4, lrb_rank=8)
    assert (z["codes"], z["W"], z["U"], z["n"]) == (128 * 32 * 128 * 64, 128 * 32 * 128 * 8 * 4,
                                                   128 * 32 * 128 * 8 * 4, 128 * 32 * 4)
    km = np.zeros((32, 128), np.uint8)
    km[:, :13] = 1
    z = sizes(B=1024, H=32, dk=128, dv=128, kind="delta", map_mode="key", map=km, hp_dtype="fp16")
    # rows padded to 4 bytes: 115 codes -> 116 bytes, 13 fp16 -> 28 bytes
    assert (z["codes"], z["hp"]) == (1024 * 32 * 128 * 116, 1024 * 32 * 128 * 28)
    # padding of rows to 4 bytes and head blocks to 16: int4, 5 quantized
    # channels -> 3 bytes -> 4 per row; 3 bf16 -> 6 bytes -> 8 per row
    km = np.zeros((2, 8), np.uint8)
    km[0, :3] = 1
    z = sizes(B=1, H=2, dk=8, dv=3, qbits=4, map_mode="key", map=km, hp_dtype="bf16")
    assert z["code_off"].tolist() == [0, 16] and z["codes"] == 16 + 16
    assert z["hp_off"].tolist() == [0, 32] and z["hp"] == 32
    km = np.zeros((1, 64), np.uint8)
    km[0, :5] = 1                      # 59 int8 codes -> 60 bytes, 5 fp16 -> 12 bytes
    z = sizes(B=2, H=1, dk=64, dv=5, map_mode="key", map=km, hp_dtype="fp16")
    assert (z["code_bstride"], z["hp_bstride"]) == (304, 64)
