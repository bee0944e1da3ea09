"""Shared test plumbing: configs for both sides from one workload, and state
conversion between the library's torch buffers and the oracle's numpy ones.
The two sides are built independently; this module only moves bytes."""
from __future__ import annotations

import numpy as np

import oracle
from quantized_recurrent_state_qstate_amd.workloads import Workload

ROUND_LIB = {"nearest": "nearest", "stochastic": "stochastic"}
ROUND_ORC = {"nearest": "rtn", "stochastic": "sr"}


def workload_map(w: Workload):
    """Precision map from the workload's statistic, built by the oracle."""
    st = w.map_stat()
    if st is None:
        return None
    stat, groups, per = st
    return oracle.build_map(stat.astype(np.float64), groups, per, w.map_frac)


def oracle_cfg(w: Workload, B=None, m=None) -> oracle.Cfg:
    if m is None:
        m = workload_map(w)
    return oracle.Cfg(kind=w.kind, decay_mode=w.decay_mode, B=w.B if B is None else B, H=w.H,
                      dk=w.dk, dv=w.dv, qbits=w.qbits, hp_dtype=w.hp_dtype, map_mode=w.map_mode,
                      map=m, rounding=ROUND_ORC[w.rounding], sr_bits=w.sr_bits, bdr=w.bdr,
                      bdr_bound=0.0, lrb_rank=w.lrb_rank, lrb_period=w.lrb_period,
                      lrb_theta=w.lrb_theta, seed=w.philox_seed, scale_dtype=w.aux_dtype, lrb_dtype=w.aux_dtype)


def lib_cfg(w: Workload, B=None, m=None):
    from quantized_recurrent_state_qstate_amd import StateConfig
    if m is None:
        m = workload_map(w)
    return StateConfig(kind=w.kind, decay_mode=w.decay_mode, B=w.B if B is None else B, H=w.H,
                       dk=w.dk, dv=w.dv, qbits=w.qbits, hp_dtype=w.hp_dtype, map_mode=w.map_mode,
                       map=m, in_dtype=w.in_dtype, rounding=ROUND_LIB[w.rounding], sr_bits=w.sr_bits,
                       bdr=w.bdr, bdr_bound=0.0, lrb_rank=w.lrb_rank, lrb_period=w.lrb_period,
                       lrb_theta=w.lrb_theta, seed=w.philox_seed, scale_dtype=w.aux_dtype,
                       lrb_dtype=w.aux_dtype)


def inputs_f32(inp: dict) -> dict:
    """Step inputs as fp32 numpy (bf16 -> fp32 is exact)."""
    out = {}
    for k, v in inp.items():
        out[k] = None if v is None else v.float().numpy()
    return out


def _np(t):
    """A device tensor's bytes as numpy (bf16 as its uint16 bit patterns)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    return t.cpu().numpy().copy()


def gpu_state_to_oracle(st: dict, hp_dtype: str) -> dict:
    """Copy the library's device buffers into the oracle's numpy layout (same bytes)."""
    codes = st["codes"].cpu().numpy().copy()
    hp_bytes = st["hp"].cpu().numpy().copy()
    hp = hp_bytes.view(np.float32) if hp_dtype == "fp32" else hp_bytes.view(np.uint16)
    return {
        "codes": codes,
        "scales": _np(st["scales"]),
        "hp": hp.copy(),
        "W": _np(st["lrb_W"]),
        "U": _np(st["lrb_U"]),
        "n": st["lrb_n"].cpu().numpy().copy(),
    }


def oracle_state_to_gpu(ost: dict, device) -> dict:
    import torch

    def dev(a):
        if a.dtype == np.uint16:   # bf16 bit patterns
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(a.copy()).to(device)
    hp = ost["hp"]
    return {
        "codes": dev(ost["codes"]),
        "scales": dev(ost["scales"]),
        "hp": torch.from_numpy(hp.view(np.uint8).copy()).to(device),
        "lrb_W": dev(ost["W"]),
        "lrb_U": dev(ost["U"]),
        "lrb_n": dev(ost["n"]),
    }


def code_values(codes_bytes: np.ndarray, qbits: int) -> np.ndarray:
    """Signed code values of a packed byte array (layout-agnostic: per byte/nibble)."""
    if qbits == 8:
        return codes_bytes.view(np.int8).astype(np.int32)
    lo = (codes_bytes & 0xF).astype(np.int32)
    hi = (codes_bytes >> 4).astype(np.int32)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    return np.stack([lo, hi], axis=-1).reshape(-1)
