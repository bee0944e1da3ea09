"""Pins of the oracle's batched step (a pool of B state slots, n sequences,
each with its own slot and step), checked against the plain step.

For each batch element b, running the plain step over the whole pool with
b's inputs placed at its slot and b's step gives, at that slot, the state
and output the batched step gives for b; slots outside the batch keep their
state, and an element whose slot is outside the pool changes nothing.  The
plain step's arithmetic is pinned elsewhere; these pins fix the slot and
step plumbing (state and random bits by slot, inputs and output by batch
position, one step per sequence)."""
import numpy as np
import pytest

import oracle

CASES = {
    "gla_key_int8_sr": dict(kind="additive", decay_mode="key", qbits=8, rounding="sr"),
    "mamba2_headmap_bf16": dict(kind="additive", decay_mode="head", qbits=8, rounding="sr", map_mode="head",
                                hp_dtype="bf16"),
    "gdn_keymap_fp16": dict(kind="delta", decay_mode="head", qbits=8, rounding="sr", map_mode="key",
                            hp_dtype="fp16"),
    "gdn_int4_lrb_bdr": dict(kind="delta", decay_mode="head", qbits=4, rounding="rtn", bdr=True, lrb_rank=3,
                             lrb_period=4),
}
B, H, DK, DV = 5, 2, 16, 12
SLOTS = np.array([3, 0, 4], np.int32)
STEPS = np.array([7, (1 << 33) + 1, 3], np.uint64)   # 3: (3+1) % 4 == 0, a merge step


def _cfg(kw, B=B):
    m = None
    if kw.get("map_mode") == "head":
        m = np.array([1, 0], np.uint8)
    elif kw.get("map_mode") == "key":
        m = (np.random.default_rng(2).random((H, DK)) < 0.3).astype(np.uint8)
    return oracle.Cfg(B=B, H=H, dk=DK, dv=DV, map=m, seed=0x5EED, **kw)


def _inputs(cfg, r, n):
    q = r.standard_normal((n, H, DK)).astype(np.float32)
    k = r.standard_normal((n, H, DK))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = r.standard_normal((n, H, DV)).astype(np.float32)
    dshape = (n, H) if cfg.decay_mode == "head" else (n, H, DK)
    d = (1 / (1 + np.exp(-r.standard_normal(dshape) - 3))).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.standard_normal((n, H))))).astype(np.float32)
    return q, k, v, d, beta


def _slot_views(cfg, st, s):
    """Every array of slot s of the pool state."""
    L = oracle.layout(cfg)
    r = cfg.lrb_rank
    hp_item = 4 if cfg.hp_dtype == "fp32" else 2
    out = {
        "codes": st["codes"][s * L["code_bstride"]:(s + 1) * L["code_bstride"]],
        "hp": st["hp"].view(np.uint8)[s * L["hp_bstride"]:(s + 1) * L["hp_bstride"]] if st["hp"].size else st["hp"],
        "scales": st["scales"][s * H * DV:(s + 1) * H * DV],
    }
    if r:
        out["W"] = st["W"][s * H * DV * r:(s + 1) * H * DV * r]
        out["U"] = st["U"][s * H * DK * r:(s + 1) * H * DK * r]
        out["n"] = st["n"][s * H:(s + 1) * H]
    del hp_item
    return out


def _warm_pool(cfg, r):
    st = oracle.new_state(cfg)
    for t in range(5):
        q, k, v, d, beta = _inputs(cfg, r, B)
        oracle.step(cfg, st, q, k, v, d, beta, step=t)
    return st


@pytest.mark.parametrize("case", list(CASES))
def test_batch_step_is_the_plain_step_at_each_slot(case):
    cfg = _cfg(CASES[case])
    r = np.random.default_rng(11)
    pool = _warm_pool(cfg, r)
    q, k, v, d, beta = _inputs(cfg, r, SLOTS.size)
    got = {n_: a.copy() for n_, a in pool.items()}
    o = oracle.step_batch(cfg, got, q, k, v, d, beta, SLOTS, STEPS)
    for b, s in enumerate(SLOTS):
        ref = {n_: a.copy() for n_, a in pool.items()}
        # pool-order inputs: element b's at slot s, anything elsewhere
        qi, ki, vi, di, bi = _inputs(cfg, np.random.default_rng(100 + b), B)
        qi[s], ki[s], vi[s], di[s], bi[s] = q[b], k[b], v[b], d[b], beta[b]
        o_ref = oracle.step(cfg, ref, qi, ki, vi, di, bi, step=int(STEPS[b]))
        np.testing.assert_array_equal(o[b], o_ref[s])
        gs, rs = _slot_views(cfg, got, s), _slot_views(cfg, ref, s)
        for name in gs:
            np.testing.assert_array_equal(gs[name], rs[name], err_msg=f"{case} slot {s} {name}")
    untouched = sorted(set(range(B)) - set(SLOTS.tolist()))
    for s in untouched:
        gs, ps = _slot_views(cfg, got, s), _slot_views(cfg, pool, s)
        for name in gs:
            np.testing.assert_array_equal(gs[name], ps[name], err_msg=f"{case} untouched slot {s} {name}")


def test_random_bits_follow_the_slot_not_the_batch_position():
    """Two batches that hold the same sequences in a different order give the
    same states and the same outputs (permuted): a sequence's rounding does
    not depend on where it sits in the batch."""
    cfg = _cfg(CASES["gla_key_int8_sr"])
    r = np.random.default_rng(5)
    pool = _warm_pool(cfg, r)
    q, k, v, d, beta = _inputs(cfg, r, 3)
    a = {n_: x.copy() for n_, x in pool.items()}
    b = {n_: x.copy() for n_, x in pool.items()}
    perm = np.array([2, 0, 1])
    oa = oracle.step_batch(cfg, a, q, k, v, d, beta, SLOTS, STEPS)
    ob = oracle.step_batch(cfg, b, q[perm], k[perm], v[perm], d[perm], beta[perm], SLOTS[perm], STEPS[perm])
    np.testing.assert_array_equal(oa[perm], ob)
    for n_ in a:
        np.testing.assert_array_equal(a[n_], b[n_])


def test_slot_outside_the_pool_is_skipped():
    cfg = _cfg(CASES["gdn_int4_lrb_bdr"])
    r = np.random.default_rng(6)
    pool = _warm_pool(cfg, r)
    q, k, v, d, beta = _inputs(cfg, r, 2)
    got = {n_: x.copy() for n_, x in pool.items()}
    out = np.full((2, H, DV), 7.0, np.float32)
    oracle.step_batch(cfg, got, q, k, v, d, beta, np.array([-1, B], np.int32), np.array([0, 0], np.uint64),
                      out=out)
    for n_ in got:
        np.testing.assert_array_equal(got[n_], pool[n_])
    assert (out == 7.0).all()
