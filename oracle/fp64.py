"""Unquantized recurrences in fp64 (TEST INFRASTRUCTURE ONLY).

These are the plain definitions of the three recurrence families the pages
name ("Gated DeltaNet, GLA, Mamba2, and RetNet" in the abstract of the page on
preserving updates), in the S[v][k] orientation (v = value / output channel,
k = key channel):

* additive (GLA per-key-channel decay; Mamba2 and RetNet scalar decay):
  S_t = S_{t-1} diag(d_t) + u_t k_t^T with u_t = beta_t v_t,  o_t = S_t q_t
* delta rule (Gated DeltaNet):
  S_t = alpha_t (S_{t-1} - beta_t S_{t-1} k_t k_t^T) + beta_t v_t k_t^T,
  o_t = S_t q_t
* delta rule with a decay per key channel (the channel-gated delta rule of
  Kimi-Linear): with D = S_{t-1} diag(d_t),
  S_t = D - beta_t (D k_t) k_t^T + beta_t v_t k_t^T; a scalar d is alpha above

Shapes: S [..., dv, dk]; q, k [..., dk]; v [..., dv]; d [...] or [..., dk];
beta, alpha [...].
"""
from __future__ import annotations

import numpy as np


def additive_step(S, q, k, v, d, beta=None):
    S = np.asarray(S, np.float64)
    d = np.asarray(d, np.float64)
    u = np.asarray(v, np.float64)
    if beta is not None:
        u = u * np.asarray(beta, np.float64)[..., None]
    dd = d[..., None, :] if d.ndim == np.asarray(k).ndim else d[..., None, None]
    S = S * dd + u[..., :, None] * np.asarray(k, np.float64)[..., None, :]
    o = np.einsum("...vk,...k->...v", S, np.asarray(q, np.float64))
    return S, o


def delta_step(S, q, k, v, alpha, beta):
    S = np.asarray(S, np.float64)
    k = np.asarray(k, np.float64)
    alpha = np.asarray(alpha, np.float64)
    b = np.asarray(beta, np.float64)[..., None, None]
    if alpha.ndim == k.ndim:              # one decay per key channel
        D = S * alpha[..., None, :]
        Dk = np.einsum("...vk,...k->...v", D, k)
        S = D - b * Dk[..., :, None] * k[..., None, :] + b * np.asarray(v, np.float64)[..., :, None] * k[..., None, :]
    else:
        a = alpha[..., None, None]
        Sk = np.einsum("...vk,...k->...v", S, k)
        S = a * (S - b * Sk[..., :, None] * k[..., None, :]) + b * np.asarray(v, np.float64)[..., :, None] * k[..., None, :]
    o = np.einsum("...vk,...k->...v", S, np.asarray(q, np.float64))
    return S, o


def run(kind, S0, qs, ks, vs, ds, betas=None):
    """Run T steps (leading axis of the per-step inputs); returns states and outputs."""
    S = np.asarray(S0, np.float64)
    states, outs = [], []
    for t in range(len(qs)):
        bt = None if betas is None else betas[t]
        if kind == "additive":
            S, o = additive_step(S, qs[t], ks[t], vs[t], ds[t], bt)
        else:
            S, o = delta_step(S, qs[t], ks[t], vs[t], ds[t], bt)
        states.append(S)
        outs.append(o)
    return states, outs
