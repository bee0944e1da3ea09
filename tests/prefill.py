"""Chunked parallel prefill of an additive gated recurrence, float64 (test
harness only): the state a serving system would hand to the decode path
after processing a prompt in chunks.

Recurrence (S[v][k]; GLA per-key decay, Mamba2 / RetNet scalar decay
broadcast over k):  S_t = S_{t-1} diag(a_t) + u_t k_t^T,  o_t = S_t q_t.

Within a chunk of C steps starting from state S0, with A_t = prod_{tau<=t} a_tau
(elementwise over k, tau from the chunk's first step):
    o_t   = S0 (A_t * q_t) + sum_{s<=t} u_s [(q_t * A_t) . (k_s / A_s)]
    S_end = S0 diag(A_C) + sum_s u_s (k_s * A_C / A_s)^T
so a chunk is two matrix products (the inter-chunk term and a masked C x C
score matrix) instead of C sequential steps.
"""
from __future__ import annotations

import numpy as np


def chunked_prefill(S0, q, k, u, a, C=16):
    """S0 [..., dv, dk]; q, k, a [T, ..., dk]; u [T, ..., dv] (u = beta v).
    Returns the state after T steps and the outputs [T, ..., dv]."""
    S = np.asarray(S0, np.float64).copy()
    q, k, u, a = (np.asarray(x, np.float64) for x in (q, k, u, a))
    T = q.shape[0]
    outs = []
    for t0 in range(0, T, C):
        qc, kc, uc, ac = q[t0:t0 + C], k[t0:t0 + C], u[t0:t0 + C], a[t0:t0 + C]
        n = qc.shape[0]
        A = np.cumprod(ac, axis=0)                                       # [n, ..., dk]
        inter = np.einsum("...vk,t...k->t...v", S, qc * A)
        scores = np.einsum("t...k,s...k->...ts", qc * A, kc / A)         # [..., n, n]
        scores = scores * np.tril(np.ones((n, n)))
        intra = np.einsum("...ts,s...v->t...v", scores, uc)
        outs.append(inter + intra)
        S = S * A[-1][..., None, :] + np.einsum("s...v,s...k->...vk", uc, kc * (A[-1] / A))
    return S, np.concatenate(outs, 0)


def sequential(S0, q, k, u, a):
    """The same recurrence one step at a time (the reference of the chunked form)."""
    S = np.asarray(S0, np.float64).copy()
    outs = []
    for t in range(q.shape[0]):
        S = S * np.asarray(a[t], np.float64)[..., None, :] + \
            np.asarray(u[t], np.float64)[..., :, None] * np.asarray(k[t], np.float64)[..., None, :]
        outs.append(np.einsum("...vk,...k->...v", S, np.asarray(q[t], np.float64)))
    return S, np.stack(outs, 0)


def workload_sequence(w, B, T):
    """q, k, u = beta v, a (decay broadcast to dk) of steps 0..T-1 of a
    workload, as float64 arrays with a leading step axis."""
    qs, ks, us, as_ = [], [], [], []
    for t in range(T):
        inp = w.step_inputs(t, B)
        q, k, v = (inp[n].double().numpy() for n in ("q", "k", "v"))
        d = inp["decay"].double().numpy()
        if d.ndim == 2:
            d = np.broadcast_to(d[..., None], k.shape)
        beta = inp["beta"]
        u = v * (beta.double().numpy()[..., None] if beta is not None else 1.0)
        qs.append(q)
        ks.append(k)
        us.append(u)
        as_.append(d)
    return np.stack(qs), np.stack(ks), np.stack(us), np.stack(as_)
