"""Brute-force pins of the oracle's Low-Rank Bypass decisions at 4 x 4.

The page on preserving updates says, in one sentence, that small updates
accumulate in a compact low-rank buffer whose sufficiently large elements are
merged into the state periodically.  The oracle implements one reading of it
in factor form (W orthonormal value basis, U key coefficients).  This file
holds a separately written simulation of the same reading that keeps the
buffer as a dense dv x dk matrix L in float64 and applies the rules to L
directly:

  1. L and the state decay on the key side: L <- L diag(d);
  2. the write vector u (additive: beta v; delta rule: beta (v - w), w the
     decayed effective state times k);
  3. while the basis has fewer than r columns, the part of u orthogonal to it
     (two Gram-Schmidt passes) joins it when its norm exceeds 2^-10 |u|;
  4. key channel k is small when |k_k| max_v |u_v| / s_v < theta (s the row
     scales on entry); a small channel adds (its in-span update) W W^T u k_k
     to L's column k and only the remainder to the state;
  5. on a merge step ((t+1) % P == 0) a column of L reaching theta s_v in
     some row moves into the state and is cleared; an all-clear buffer
     empties the basis;
  6. the readout is (S_pre + L) q.

Teacher-forced: every step starts from the oracle's stored state, and the
simulation's small-channel set, basis growth and merge set must equal the
decisions the oracle reports for that step; its S_pre, buffer and output must
equal the oracle's to fp32 accuracy.  Planted mistakes in copies of the oracle
(the LSB taken after the step instead of on entry, the minimum over rows
instead of the maximum, the smallness comparison reversed, a merge that needs
every row, a merge clock off by one) each fail these checks.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

DK = DV = 4
T = 12
THETA = 0.5


def _inputs(kind, decay_mode, r, B, H):
    q = r.standard_normal((B, H, DK))
    k = r.standard_normal((B, H, DK))
    if kind == "delta":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k[..., DK // 2:] *= 0.08                   # half the key channels carry small updates
    # in head 0 the other half is bounded away from zero (never small), so its
    # buffer can clear completely at a merge and the basis resets
    k[:, 0, :DK // 2] = np.sign(k[:, 0, :DK // 2]) * (1 + np.abs(k[:, 0, :DK // 2]))
    v = r.standard_normal((B, H, DV))
    shape = (B, H, DK) if decay_mode == "key" else (B, H)
    d = 1 / (1 + np.exp(-(r.standard_normal(shape) + 2.5)))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, H)))) if kind == "delta" else None
    f = np.float32
    return (q.astype(f), k.astype(f), v.astype(f), d.astype(f), None if beta is None else beta.astype(f))


def _decode(cfg, st):
    """Stored state -> per head: dequantized state [dv,dk], scales, W, U, n
    (float64), read from the documented byte layout."""
    L = oracle.layout(cfg)
    rb = ((DK * cfg.qbits + 7) // 8 + 3) // 4 * 4
    r = cfg.lrb_rank
    heads = []
    for bh in range(cfg.B * cfg.H):
        b, h = divmod(bh, cfg.H)
        base = b * L["code_bstride"] + int(L["code_off"][h])
        s = st["scales"][bh * DV:(bh + 1) * DV].astype(np.float64)
        codes = np.zeros((DV, DK))
        for v in range(DV):
            row = st["codes"][base + v * rb: base + v * rb + rb]
            if cfg.qbits == 8:
                c = row[:DK].view(np.int8).astype(np.int64)
            else:
                nib = np.stack([row & 0xF, row >> 4], 1).reshape(-1)[:DK].astype(np.int64)
                c = np.where(nib >= 8, nib - 16, nib)
            codes[v] = c
        W = st["W"][bh * DV * r:(bh + 1) * DV * r].reshape(DV, r).astype(np.float64)
        U = st["U"][bh * DK * r:(bh + 1) * DK * r].reshape(DK, r).astype(np.float64)
        heads.append(dict(Sh=s[:, None] * codes, s=s, W=W, U=U, n=int(st["n"][bh])))
    return heads


def _simulate(cfg, hd, q, k, v, d, beta, t):
    """One step of the dense-buffer reading for one head (float64).  Returns
    the decisions, S_pre, the buffer after the step, the output, and the
    smallest relative distance of any decision from its threshold."""
    n, r = hd["n"], cfg.lrb_rank
    W = hd["W"][:, :n]
    Lb = W @ hd["U"][:, :n].T
    dvec = d if d.ndim == 1 else np.full(DK, float(d))
    Ld = Lb * dvec[None, :]
    Sd = hd["Sh"] * dvec[None, :]
    bt = 1.0 if beta is None else float(beta)
    if cfg.kind == "additive":
        u = bt * v
    else:
        u = bt * (v - (Sd @ k + Ld @ k))
    margin = np.inf
    grown = False
    if n < r:
        y = u.copy()
        for _ in range(2):
            for j in range(W.shape[1]):
                y = y - (W[:, j] @ y) * W[:, j]
        ny, lim = np.linalg.norm(y), 2.0 ** -10 * np.linalg.norm(u)
        margin = min(margin, abs(ny - lim) / max(lim, 1e-300))
        if ny > lim:
            W = np.concatenate([W, (y / ny)[:, None]], 1)
            grown = True
    c = W.T @ u
    upar = W @ c
    uperp = u - upar
    s = hd["s"]
    with np.errstate(divide="ignore", invalid="ignore"):
        gv = np.where(s > 0, np.abs(u) / np.where(s > 0, s, 1), np.where(np.abs(u) > 0, np.inf, 0.0))
    g = gv.max()
    small = np.zeros(DK, bool)
    if np.isfinite(g):
        x = np.abs(k) * g
        small = x < THETA
        margin = min(margin, (np.abs(x - THETA) / THETA).min())
    Lp = Ld + np.outer(upar, k * small)
    Sp = Sd + np.outer(u, k * ~small) + np.outer(uperp, k * small)
    merged = np.zeros(DK, bool)
    n_after = W.shape[1]
    if (t + 1) % cfg.lrb_period == 0:
        lim = THETA * s[:, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            rel = np.where(lim > 0, np.abs(Lp) / np.where(lim > 0, lim, 1), np.inf)
        nz = Lp != 0
        merged = (nz & (rel >= 1)).any(0)
        for kk in range(DK):   # a column's largest row ratio decides it
            if nz[:, kk].any():
                margin = min(margin, abs(rel[nz[:, kk], kk].max() - 1))
        Sp[:, merged] += Lp[:, merged]
        Lp[:, merged] = 0.0
        if not Lp.any():
            n_after = 0
    o = Sp @ q + Lp @ q
    return dict(small=small, merged=merged, grown=grown, n_after=n_after, Sp=Sp, L=Lp, o=o, margin=margin)


def _run(kind, decay_mode, rank, period, seed, stats):
    """Teacher-forced run against the oracle loaded now; returns mismatches
    (empty when every decision and value agrees)."""
    B, H = 1, 3
    cfg = oracle.Cfg(kind=kind, decay_mode=decay_mode, B=B, H=H, dk=DK, dv=DV, qbits=4, rounding="rtn", bdr=True,
                     lrb_rank=rank, lrb_period=period, lrb_theta=THETA, seed=3)
    rng = np.random.default_rng(seed)
    st = oracle.new_state(cfg)
    oracle.quantize(cfg, (1.5 * rng.standard_normal((B, H, DV, DK))).astype(np.float32), st)
    bad = []
    for t in range(T):
        q, k, v, d, beta = _inputs(kind, decay_mode, rng, B, H)
        before = _decode(cfg, st)
        o, sp, small, merged, nb, na = oracle.step_lrb_trace(cfg, st, q, k, v, d, beta, step=t)
        after = _decode(cfg, st)
        for bh in range(B * H):
            b, h = divmod(bh, H)
            sim = _simulate(cfg, before[bh], q[b, h].astype(np.float64), k[b, h].astype(np.float64),
                            v[b, h].astype(np.float64), d[b, h].astype(np.float64),
                            None if beta is None else beta[b, h], t)
            where = f"{kind}/{decay_mode} r={rank} P={period} seed={seed} t={t} head={bh}"
            if sim["margin"] < 1e-5:
                stats["marginal"] += 1
                continue
            if not np.array_equal(sim["small"], small[b, h]):
                bad.append(f"{where}: small {small[b, h].astype(int)} vs simulated {sim['small'].astype(int)}")
            if sim["n_after"] > 0 and sim["grown"] != (na[b, h] == nb[b, h] + 1):   # no reset: n tells growth
                bad.append(f"{where}: basis {nb[b, h]}->{na[b, h]}, simulated growth {sim['grown']}")
            if sim["n_after"] != na[b, h]:
                bad.append(f"{where}: basis size {na[b, h]} vs simulated {sim['n_after']}")
            if not np.array_equal(sim["merged"], merged[b, h]):
                bad.append(f"{where}: merged {merged[b, h].astype(int)} vs simulated {sim['merged'].astype(int)}")
            scale = np.abs(sim["Sp"]).max() + np.abs(sim["L"]).max() + 1e-30
            Lo = after[bh]["W"][:, :na[b, h]] @ after[bh]["U"][:, :na[b, h]].T
            for name, got, want in (("S_pre", sp[b, h], sim["Sp"]), ("buffer", Lo, sim["L"]),
                                    ("output", o[b, h], sim["o"])):
                tol = 2e-5 * (scale * (np.abs(q[b, h]).sum() if name == "output" else 1.0))
                err = np.abs(np.asarray(got, np.float64) - want).max()
                if err > tol:
                    bad.append(f"{where}: {name} off by {err:.3g} (tolerance {tol:.3g})")
            stats["small"] += int(sim["small"].sum())
            stats["large"] += int((~sim["small"]).sum())
            stats["grown"] += int(sim["grown"])
            stats["merged"] += int(sim["merged"].sum())
            if (t + 1) % period == 0:
                stats["kept"] += int((~sim["merged"]).sum())
            stats["reset"] += int(nb[b, h] > 0 and na[b, h] == 0)
    return bad


CASES = [(kind, dm, rank, period) for kind in ("additive", "delta") for dm in ("key", "head")
         for rank in (1, 2) for period in (2, 3)]


def _all_mismatches(stats):
    bad = []
    for kind, dm, rank, period in CASES:
        for seed in (1, 2):
            bad += _run(kind, dm, rank, period, seed, stats)
    return bad


def _stats():
    return dict(small=0, large=0, grown=0, merged=0, kept=0, reset=0, marginal=0)


def test_lrb_decisions_match_dense_simulation():
    stats = _stats()
    bad = _all_mismatches(stats)
    assert not bad, "\n".join(bad[:10])
    # every rule fired both ways, and no decision sat on its threshold
    assert stats["small"] > 50 and stats["large"] > 50, stats
    assert stats["grown"] > 20 and stats["merged"] > 20 and stats["kept"] > 20, stats
    assert stats["reset"] > 0, stats
    assert stats["marginal"] == 0, stats


# Planted mistakes, each a text substitution in a copy of the oracle's source.
_PHASE_CALL = "    lrb_phase(c, W, U, &st->n[bh], u, kh, s_old, step, small, u_perp, merged, mflag);\n"
_MERGE_TEST = "        if (col != 0.0f && fabsf(col) >= theta * s_old[v]) big = 1;\n"
MUTANTS = {
    # the LSB of the smallness and merge tests taken from the row's scale
    # after the step (its maximum of the plain update over Q) instead of on entry
    "lsb_after_step": (_PHASE_CALL,
                       "    float* lsb = (float*)malloc(sizeof(float) * (size_t)dv);\n"
                       "    for (int v = 0; v < dv; ++v) {\n"
                       "      float m = 0.0f;\n"
                       "      for (int k = 0; k < dk; ++k) {\n"
                       "        float x = fabsf(fmaf(u[v], kh[k], d[k] * sh[v * dk + k]));\n"
                       "        if (x > m) m = x;\n"
                       "      }\n"
                       "      lsb[v] = m / ((c->qbits == 8) ? 127.0f : 7.0f);\n"
                       "    }\n"
                       "    lrb_phase(c, W, U, &st->n[bh], u, kh, lsb, step, small, u_perp, merged, mflag);\n"
                       "    free(lsb);\n"),
    # the smallest row ratio instead of the largest
    "min_over_rows": ("    if (gv > g) g = gv;\n", "    if (v == 0 || gv < g) g = gv;\n"),
    # the smallness comparison reversed
    "smallness_reversed": ("(fabsf(kk[k]) * g < theta)", "(fabsf(kk[k]) * g >= theta)"),
    # a merge that needs every row to reach the threshold
    "merge_every_row": (_MERGE_TEST, "        if (!(col != 0.0f && fabsf(col) >= theta * s_old[v])) big = 0;\n"),
    # merge clock off by one step
    "merge_clock": ("((step + 1u) % (uint64_t)c->lrb_period) == 0u", "(step % (uint64_t)c->lrb_period) == 0u"),
}


def _build_mutant(tmp, name):
    here = os.path.dirname(oracle.__file__)
    src = open(os.path.join(here, "qs_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site of {name} not found once in the oracle"
    if name == "merge_every_row":
        src = src.replace("      int big = 0;\n      for (int v = 0; v < dv; ++v) {\n        float col",
                          "      int big = 1;\n      for (int v = 0; v < dv; ++v) {\n        float col")
    src = src.replace(old, new)
    cpath = os.path.join(tmp, f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    import shutil
    shutil.copy(os.path.join(here, "qs_oracle.h"), tmp)
    so = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-I", tmp, cpath, "-o", so, "-lm"], check=True, capture_output=True)
    return so


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(tmp, name)
        with oracle.using(so):
            bad = _all_mismatches(_stats())
    assert bad, f"the simulation did not catch the planted mistake {name}"
