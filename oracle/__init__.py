"""CPU oracle for the quantized recurrent-state decode step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg load this package; the library never does.
It shares no code with the HIP library.

``qs_oracle.c`` holds the quantized step (plain scalar C, fp32 element
arithmetic, fp64 reductions); ``fp64.py`` holds the unquantized recurrences
in fp64.  This module is argument marshalling over ctypes plus numpy
allocation of the stored-state buffers in the documented layout.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

from . import build as _build

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        _LIB = configure(ctypes.CDLL(_build.build()))
    return _LIB


@contextlib.contextmanager
def using(path: str):
    """Run the wrappers below against another build of the oracle's source
    (tests that plant a mistake in a copy of it, on the CPU)."""
    global _LIB
    saved = _LIB
    _LIB = configure(ctypes.CDLL(path))
    try:
        yield _LIB
    finally:
        _LIB = saved


def configure(L):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.POINTER
    c_cfg = P(_Cfg)
    L.orc_layout.argtypes = [c_cfg, P(_Sizes), P(ctypes.c_uint64), P(ctypes.c_uint64),
                             P(ctypes.c_int32)]
    L.orc_layout.restype = ctypes.c_int
    L.orc_philox4x32_10.argtypes = [P(ctypes.c_uint32), P(ctypes.c_uint32), P(ctypes.c_uint32)]
    L.orc_philox4x32_10.restype = None
    L.orc_random_bits.argtypes = [c_cfg, ctypes.c_uint64, ctypes.c_uint64]
    L.orc_random_bits.restype = ctypes.c_uint32
    L.orc_sr_round.argtypes = [ctypes.c_float, ctypes.c_uint32, ctypes.c_int32]
    L.orc_sr_round.restype = ctypes.c_float
    L.orc_inv_rtz.argtypes = [ctypes.c_float, ctypes.c_float]
    L.orc_inv_rtz.restype = ctypes.c_float
    L.orc_scale_bf16_up.argtypes = [ctypes.c_float, ctypes.c_float]
    L.orc_scale_bf16_up.restype = ctypes.c_float
    L.orc_to_bf16.argtypes = [ctypes.c_float]
    L.orc_to_bf16.restype = ctypes.c_uint16
    L.orc_to_fp16.argtypes = [ctypes.c_float]
    L.orc_to_fp16.restype = ctypes.c_uint16
    L.orc_from_bf16.argtypes = [ctypes.c_uint16]
    L.orc_from_bf16.restype = ctypes.c_float
    L.orc_from_fp16.argtypes = [ctypes.c_uint16]
    L.orc_from_fp16.restype = ctypes.c_float
    L.orc_build_map.argtypes = [P(ctypes.c_double), ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_double, P(ctypes.c_uint8)]
    L.orc_build_map.restype = ctypes.c_int
    L.orc_quantize.argtypes = [c_cfg, P(ctypes.c_float), P(_State), ctypes.c_uint64]
    L.orc_quantize.restype = ctypes.c_int
    L.orc_dequantize.argtypes = [c_cfg, P(_State), P(ctypes.c_float)]
    L.orc_dequantize.restype = ctypes.c_int
    fp = P(ctypes.c_float)
    L.orc_step.argtypes = [c_cfg, P(_State), fp, fp, fp, fp, fp, fp, ctypes.c_uint64, fp,
                           P(ctypes.c_int64), ctypes.c_int64]
    L.orc_step.restype = ctypes.c_int
    L.orc_step_batch.argtypes = [c_cfg, P(_State), fp, fp, fp, fp, fp, fp, ctypes.c_int32,
                                 P(ctypes.c_int32), P(ctypes.c_uint64)]
    L.orc_step_batch.restype = ctypes.c_int
    L.orc_step_lrb_trace.argtypes = [c_cfg, P(_State), fp, fp, fp, fp, fp, fp, ctypes.c_uint64, fp,
                                     P(_Trace)]
    L.orc_step_lrb_trace.restype = ctypes.c_int
    return L


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("decay_mode", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("qbits", ctypes.c_int32), ("hp_dtype", ctypes.c_int32), ("map_mode", ctypes.c_int32),
        ("map", ctypes.POINTER(ctypes.c_uint8)), ("rounding", ctypes.c_int32),
        ("sr_bits", ctypes.c_int32), ("bdr", ctypes.c_int32), ("bdr_bound", ctypes.c_float),
        ("lrb_rank", ctypes.c_int32), ("lrb_period", ctypes.c_int32), ("lrb_theta", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("scale_dtype", ctypes.c_int32), ("lrb_dtype", ctypes.c_int32),
        ("scale_axis", ctypes.c_int32),
    ]


class _Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("codes", "scales", "hp", "W", "U", "n", "code_bstride", "hp_bstride")]


class _State(ctypes.Structure):
    _fields_ = [("codes", ctypes.POINTER(ctypes.c_uint8)), ("scales", ctypes.c_void_p),
                ("hp", ctypes.c_void_p), ("W", ctypes.c_void_p),
                ("U", ctypes.c_void_p), ("n", ctypes.POINTER(ctypes.c_int32))]


class _Trace(ctypes.Structure):
    _fields_ = [("small", ctypes.POINTER(ctypes.c_int32)), ("merged", ctypes.POINTER(ctypes.c_int32)),
                ("n_before", ctypes.POINTER(ctypes.c_int32)), ("n_after", ctypes.POINTER(ctypes.c_int32))]


KIND = {"additive": 0, "delta": 1}
DECAY = {"head": 0, "key": 1}
HP = {"fp32": 0, "bf16": 1, "fp16": 2}
MAP = {"none": 0, "head": 1, "key": 2}
ROUND = {"rtn": 0, "sr": 1}
SDT = {"fp32": 0, "bf16": 1}
AXIS = {"value": 0, "key": 1, "head": 2}


@dataclasses.dataclass
class Cfg:
    """Oracle configuration (its own definition; see qs_oracle.h)."""
    kind: str = "additive"
    decay_mode: str = "head"
    B: int = 1
    H: int = 1
    dk: int = 64
    dv: int = 64
    qbits: int = 8
    hp_dtype: str = "bf16"
    map_mode: str = "none"
    map: Optional[np.ndarray] = None
    rounding: str = "sr"
    sr_bits: int = 16
    bdr: bool = False
    bdr_bound: float = 0.0
    lrb_rank: int = 0
    lrb_period: int = 64
    lrb_theta: float = 0.5
    seed: int = 0
    scale_dtype: str = "fp32"   # fp32 | bf16
    lrb_dtype: str = "fp32"     # fp32 | bf16
    scale_axis: str = "value"   # value | key | head

    def c(self) -> _Cfg:
        s = _Cfg()
        s.kind, s.decay_mode = KIND[self.kind], DECAY[self.decay_mode]
        s.B, s.H, s.dk, s.dv = self.B, self.H, self.dk, self.dv
        s.qbits, s.hp_dtype, s.map_mode = self.qbits, HP[self.hp_dtype], MAP[self.map_mode]
        if self.map is not None:
            # converted once per map object and kept: threads that share a Cfg
            # must not free the array another thread's call is reading
            keep = getattr(self, "_map_keep", None)
            if keep is None or keep[0] is not self.map:
                keep = (self.map, np.ascontiguousarray(self.map, dtype=np.uint8))
                self._map_keep = keep
            s.map = keep[1].ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        s.rounding, s.sr_bits = ROUND[self.rounding], self.sr_bits
        s.bdr, s.bdr_bound = int(self.bdr), self.bdr_bound
        s.lrb_rank, s.lrb_period, s.lrb_theta = self.lrb_rank, self.lrb_period, self.lrb_theta
        s.seed = self.seed
        s.scale_dtype, s.lrb_dtype = SDT[self.scale_dtype], SDT[self.lrb_dtype]
        s.scale_axis = AXIS[self.scale_axis]
        return s


def _fp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def layout(cfg: Cfg) -> dict:
    c = cfg.c()
    s = _Sizes()
    co = np.zeros(cfg.H, np.uint64)
    ho = np.zeros(cfg.H, np.uint64)
    nq = np.zeros(cfg.H, np.int32)
    rc = lib().orc_layout(ctypes.byref(c), ctypes.byref(s),
                          co.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                          ho.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                          nq.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc:
        raise ValueError("oracle: invalid configuration")
    out = {n: int(getattr(s, n)) for n, _ in _Sizes._fields_}
    out.update(code_off=co, hp_off=ho, nq=nq)
    return out


def new_state(cfg: Cfg) -> dict:
    """Zero-filled stored state (the zero state S = 0) in the documented layout."""
    L = layout(cfg)
    hp_dt = np.float32 if cfg.hp_dtype == "fp32" else np.uint16
    hp_item = 4 if cfg.hp_dtype == "fp32" else 2
    s_dt = np.float32 if cfg.scale_dtype == "fp32" else np.uint16     # bf16: raw bits
    l_dt = np.float32 if cfg.lrb_dtype == "fp32" else np.uint16
    return {
        "codes": np.zeros(L["codes"], np.uint8),
        "scales": np.zeros(L["scales"] // np.dtype(s_dt).itemsize, s_dt),
        "hp": np.zeros(L["hp"] // hp_item, hp_dt),
        "W": np.zeros(L["W"] // np.dtype(l_dt).itemsize, l_dt),
        "U": np.zeros(L["U"] // np.dtype(l_dt).itemsize, l_dt),
        "n": np.zeros(L["n"] // 4, np.int32),
    }


def widen(a: np.ndarray) -> np.ndarray:
    """A stored scale or buffer array as float64 (bf16 bits widened exactly)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _state_struct(st: dict) -> _State:
    s = _State()
    for key in ("codes", "scales", "hp", "W", "U", "n"):
        a = st[key]
        assert a.flags.c_contiguous
    s.codes = st["codes"].ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    s.scales = st["scales"].ctypes.data_as(ctypes.c_void_p)
    s.hp = st["hp"].ctypes.data_as(ctypes.c_void_p)
    s.W = st["W"].ctypes.data_as(ctypes.c_void_p)
    s.U = st["U"].ctypes.data_as(ctypes.c_void_p)
    s.n = st["n"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return s


def _f32(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None:
        assert a.size == int(np.prod(shape)), (a.shape, shape)
    return a


def quantize(cfg: Cfg, S: np.ndarray, st: dict, step: int = 0) -> None:
    S = _f32(S, (cfg.B, cfg.H, cfg.dv, cfg.dk))
    c = cfg.c()
    s = _state_struct(st)
    if lib().orc_quantize(ctypes.byref(c), _fp(S), ctypes.byref(s), step):
        raise ValueError("oracle quantize failed")


def dequantize(cfg: Cfg, st: dict) -> np.ndarray:
    S = np.zeros((cfg.B, cfg.H, cfg.dv, cfg.dk), np.float32)
    c = cfg.c()
    s = _state_struct(st)
    if lib().orc_dequantize(ctypes.byref(c), ctypes.byref(s), _fp(S)):
        raise ValueError("oracle dequantize failed")
    return S


def step(cfg: Cfg, st: dict, q, k, v, decay, beta=None, step: int = 0, heads=None,
         want_sp: bool = False, out=None):
    """One decode step in place on ``st``; returns o [B,H,dv] (and S_pre)."""
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = _f32(q, (B, H, dk))
    k = _f32(k, (B, H, dk))
    v = _f32(v, (B, H, dv))
    decay = _f32(decay, (B, H) if cfg.decay_mode == "head" else (B, H, dk))
    beta_p = None
    if beta is not None:
        beta = _f32(beta, (B, H))
        beta_p = _fp(beta)
    if out is None:
        out = np.zeros((B, H, dv), np.float32)
    sp = np.zeros((B, H, dv, dk), np.float32) if want_sp else None
    hp_ = None
    nh = 0
    if heads is not None:
        heads = np.ascontiguousarray(heads, dtype=np.int64)
        hp_ = heads.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        nh = heads.size
    c = cfg.c()
    s = _state_struct(st)
    rc = lib().orc_step(ctypes.byref(c), ctypes.byref(s), _fp(q), _fp(k), _fp(v), _fp(decay),
                        beta_p, _fp(out), step, _fp(sp) if sp is not None else None, hp_, nh)
    if rc:
        raise ValueError("oracle step failed")
    return (out, sp) if want_sp else out


def step_lrb_trace(cfg: Cfg, st: dict, q, k, v, decay, beta=None, step: int = 0):
    """One step of every head (low-rank bypass on), in place on ``st``.
    Returns o [B,H,dv], S_pre [B,H,dv,dk] and the buffer decisions: small and
    merged [B,H,dk] (bool), basis size before and after [B,H]."""
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = _f32(q, (B, H, dk))
    k = _f32(k, (B, H, dk))
    v = _f32(v, (B, H, dv))
    decay = _f32(decay, (B, H) if cfg.decay_mode == "head" else (B, H, dk))
    beta_p = None
    if beta is not None:
        beta = _f32(beta, (B, H))
        beta_p = _fp(beta)
    out = np.zeros((B, H, dv), np.float32)
    sp = np.zeros((B, H, dv, dk), np.float32)
    small = np.zeros((B, H, dk), np.int32)
    merged = np.zeros((B, H, dk), np.int32)
    nb = np.zeros((B, H), np.int32)
    na = np.zeros((B, H), np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    tr = _Trace(small.ctypes.data_as(ip), merged.ctypes.data_as(ip), nb.ctypes.data_as(ip), na.ctypes.data_as(ip))
    c = cfg.c()
    s = _state_struct(st)
    rc = lib().orc_step_lrb_trace(ctypes.byref(c), ctypes.byref(s), _fp(q), _fp(k), _fp(v), _fp(decay), beta_p,
                                  _fp(out), step, _fp(sp), ctypes.byref(tr))
    if rc:
        raise ValueError("oracle traced step failed")
    return out, sp, small.astype(bool), merged.astype(bool), nb, na


def step_batch(cfg: Cfg, st: dict, q, k, v, decay, beta, slot, steps, out=None):
    """A step for n = len(slot) sequences whose states sit in slots of ``st``
    (the config's B states); inputs [n,H,...]; element b uses state slot
    slot[b] and step steps[b].  Returns o [n,H,dv]."""
    H, dk, dv = cfg.H, cfg.dk, cfg.dv
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    steps = np.ascontiguousarray(steps, dtype=np.uint64)
    n = slot.size
    q = _f32(q, (n, H, dk))
    k = _f32(k, (n, H, dk))
    v = _f32(v, (n, H, dv))
    decay = _f32(decay, (n, H) if cfg.decay_mode == "head" else (n, H, dk))
    beta_p = None
    if beta is not None:
        beta = _f32(beta, (n, H))
        beta_p = _fp(beta)
    if out is None:
        out = np.zeros((n, H, dv), np.float32)
    c = cfg.c()
    s = _state_struct(st)
    rc = lib().orc_step_batch(ctypes.byref(c), ctypes.byref(s), _fp(q), _fp(k), _fp(v), _fp(decay), beta_p,
                              _fp(out), n, slot.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                              steps.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    if rc:
        raise ValueError("oracle batch step failed")
    return out


def philox(ctr, key):
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    kk = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, kk, o)
    return [int(x) for x in o]


def random_bits(cfg: Cfg, e: int, step: int) -> int:
    c = cfg.c()
    return int(lib().orc_random_bits(ctypes.byref(c), e, step))


def sr_round(x: float, u: int, sr_bits: int = 16) -> float:
    return float(lib().orc_sr_round(x, u, sr_bits))


def inv_rtz(q: float, m: float) -> float:
    """q / m rounded toward zero to fp32 (q, m > 0, finite quotient)."""
    return float(lib().orc_inv_rtz(q, m))


def scale_bf16_up(m: float, q: float) -> float:
    """Smallest bf16 value s with q s >= m (the rounded-up bf16 row scale)."""
    return float(lib().orc_scale_bf16_up(m, q))


def to_bf16(x: float) -> int:
    return int(lib().orc_to_bf16(x))


def to_fp16(x: float) -> int:
    return int(lib().orc_to_fp16(x))


def from_bf16(h: int) -> float:
    return float(lib().orc_from_bf16(h))


def from_fp16(h: int) -> float:
    return float(lib().orc_from_fp16(h))


def build_map(stat: np.ndarray, groups: int, per_group: int, frac: float) -> np.ndarray:
    stat = np.ascontiguousarray(stat, dtype=np.float64)
    assert stat.size == groups * per_group
    m = np.zeros(groups * per_group, np.uint8)
    rc = lib().orc_build_map(stat.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), groups,
                             per_group, frac, m.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    if rc:
        raise ValueError("oracle build_map failed")
    return m
