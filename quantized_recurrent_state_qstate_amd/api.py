"""Python front end of libqstate: a handle plus torch-owned device buffers.

torch provides device memory and streams only; every computation of the
decode path (dequantize, decay + update, readout, requantize) runs in the
library's kernels through the C ABI of include/qstate.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np

from . import _lib


@dataclasses.dataclass
class StateConfig:
    """Mirror of qstate_config with readable enumerations."""
    kind: str = "additive"          # additive | delta
    decay_mode: str = "head"        # head | key
    B: int = 1
    H: int = 1
    dk: int = 128
    dv: int = 128
    qbits: int = 8                  # 8 | 4
    hp_dtype: str = "bf16"          # fp32 | bf16 | fp16
    map_mode: str = "none"          # none | head | key
    map: Optional[np.ndarray] = None
    in_dtype: str = "bf16"          # fp32 | bf16
    rounding: str = "stochastic"    # nearest | stochastic
    sr_bits: int = 16
    bdr: bool = False
    bdr_bound: float = 0.0
    lrb_rank: int = 0
    lrb_period: int = 64
    lrb_theta: float = 0.5
    seed: int = 0
    scale_dtype: str = "fp32"       # fp32 | bf16 (bf16: with lrb_dtype bf16 and the low-rank bypass)
    lrb_dtype: str = "fp32"         # fp32 | bf16
    scale_axis: str = "value"       # value | key | head (key and head: ablations, map none, no buffer)

    def to_c(self) -> _lib.Config:
        c = _lib.Config()
        c.abi_version = _lib.ABI_VERSION
        c.kind = _lib.KIND[self.kind]
        c.decay_mode = _lib.DECAY[self.decay_mode]
        c.B, c.H, c.dk, c.dv = self.B, self.H, self.dk, self.dv
        c.qbits = self.qbits
        c.hp_dtype = _lib.DTYPE[self.hp_dtype]
        c.map_mode = _lib.MAP[self.map_mode]
        if self.map is not None:
            self._map_keep = np.ascontiguousarray(self.map, dtype=np.uint8).ravel()
            c.map = self._map_keep.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        c.in_dtype = _lib.DTYPE[self.in_dtype]
        c.rounding = _lib.ROUNDING[self.rounding]
        c.sr_bits = self.sr_bits
        c.bdr = int(self.bdr)
        c.bdr_bound = self.bdr_bound
        c.lrb_rank, c.lrb_period, c.lrb_theta = self.lrb_rank, self.lrb_period, self.lrb_theta
        c.seed = self.seed
        c.scale_dtype = _lib.DTYPE[self.scale_dtype]
        c.lrb_dtype = _lib.DTYPE[self.lrb_dtype]
        c.scale_axis = _lib.AXIS[self.scale_axis]
        return c


def plan(cfg: StateConfig) -> dict:
    """Buffer sizes in bytes (host only; no GPU needed)."""
    c = cfg.to_c()
    s = _lib.Sizes()
    _lib.check(_lib.lib().qstate_plan(ctypes.byref(c), ctypes.byref(s)), "qstate_plan")
    return {n: int(getattr(s, n)) for n, _ in _lib.Sizes._fields_}


def build_map(stat, groups: int, per_group: int, frac: float) -> np.ndarray:
    """Decay-based mixed-precision map: smallest decay-rate units flagged (host)."""
    stat = np.ascontiguousarray(stat, dtype=np.float32).ravel()
    assert stat.size == groups * per_group
    m = np.zeros(groups * per_group, np.uint8)
    _lib.check(_lib.lib().qstate_build_map(stat.ctypes.data, groups, per_group, frac, m.ctypes.data),
               "qstate_build_map")
    return m


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _state_dtypes(cfg: "StateConfig") -> dict:
    """torch dtype name of each state buffer (bf16 scales and factors in the bf16 layout)."""
    sd = "bfloat16" if cfg.scale_dtype == "bf16" else "float32"
    ld = "bfloat16" if cfg.lrb_dtype == "bf16" else "float32"
    return {"codes": "uint8", "scales": sd, "hp": "uint8", "lrb_W": ld, "lrb_U": ld, "lrb_n": "int32"}


def check_tensor(name: str, t, dtype, numel: int, device, at_least: bool = False) -> None:
    """Host-side argument check before a pointer crosses the C ABI: the kernels
    read and write exactly the planned extents, so a tensor of the wrong dtype,
    size, memory layout or device would make them read or write out of bounds
    or get wrong results.  Raises ValueError (checks in that order)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if (t.numel() < numel) if at_least else (t.numel() != numel):
        raise ValueError(f"{name}: {t.numel()} elements, expected {'at least ' if at_least else ''}{numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def check_state(cfg: "StateConfig", sizes: dict, st: dict, device) -> None:
    """Every buffer the plan sizes > 0 must be present, typed and large enough."""
    import torch
    for n, dt in _state_dtypes(cfg).items():
        nbytes = sizes[n]
        if nbytes == 0:
            continue
        dtype = getattr(torch, dt)
        item = torch.empty((), dtype=dtype).element_size()
        check_tensor(f"state[{n!r}]", st.get(n), dtype, nbytes // item, device, at_least=True)


def check_inputs(cfg: "StateConfig", n: int, device, q, k, v, decay, beta, out) -> None:
    """Inputs of a step for n batch elements: q, k [n,H,dk] and v [n,H,dv] in
    the configured input dtype, decay fp32 [n,H] (or [n,H,dk] per key), beta
    fp32 [n,H] or None, out fp32 [n,H,dv]."""
    import torch
    ind = torch.bfloat16 if cfg.in_dtype == "bf16" else torch.float32
    nh = n * cfg.H
    check_tensor("q", q, ind, nh * cfg.dk, device)
    check_tensor("k", k, ind, nh * cfg.dk, device)
    check_tensor("v", v, ind, nh * cfg.dv, device)
    check_tensor("decay", decay, torch.float32, nh * (cfg.dk if cfg.decay_mode == "key" else 1), device)
    if beta is not None:
        check_tensor("beta", beta, torch.float32, nh, device)
    check_tensor("out", out, torch.float32, nh * cfg.dv, device)


class QState:
    """A libqstate handle for one configuration on the current HIP device."""

    def __init__(self, cfg: StateConfig):
        import torch
        self.cfg = cfg
        self._c = cfg.to_c()
        self._h = ctypes.c_void_p()
        s = _lib.Sizes()
        _lib.check(_lib.lib().qstate_init(ctypes.byref(self._c), ctypes.byref(self._h), ctypes.byref(s)),
                   "qstate_init")
        self.sizes = {n: int(getattr(s, n)) for n, _ in _lib.Sizes._fields_}
        self.device = torch.device("cuda", torch.cuda.current_device())

    def close(self) -> None:
        if self._h:
            _lib.lib().qstate_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def kernel_name(self) -> str:
        return _lib.lib().qstate_kernel_name(self._h).decode()

    def new_state(self) -> dict:
        """Zero-filled state buffers (the state S = 0), owned by torch."""
        import torch
        z = self.sizes
        dev = self.device

        def buf(nbytes, dtype, item):
            return torch.zeros(max(nbytes // item, 1 if nbytes else 0), dtype=dtype, device=dev)

        dts = {n: getattr(torch, d) for n, d in _state_dtypes(self.cfg).items()}
        return {n: buf(z[n], dts[n], torch.empty((), dtype=dts[n]).element_size()) for n in dts}

    @staticmethod
    def _tensors(st: dict) -> _lib.Tensors:
        t = _lib.Tensors()
        for n in ("codes", "scales", "hp", "lrb_W", "lrb_U", "lrb_n"):
            x = st.get(n)
            setattr(t, n, x.data_ptr() if (x is not None and x.numel() > 0) else None)
        return t

    @staticmethod
    def _stream(stream) -> Optional[int]:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        return stream.cuda_stream

    def quantize(self, S, st: dict, step: int = 0, stream=None) -> None:
        import torch
        c = self.cfg
        check_tensor("S", S, torch.float32, c.B * c.H * c.dv * c.dk, self.device)
        check_state(c, self.sizes, st, self.device)
        t = self._tensors(st)
        _lib.check(_lib.lib().qstate_quantize(self._h, _ptr(S), ctypes.byref(t), step, self._stream(stream)),
                   "qstate_quantize")

    def dequantize(self, st: dict, out=None, stream=None):
        import torch
        c = self.cfg
        if out is None:
            out = torch.empty((c.B, c.H, c.dv, c.dk), dtype=torch.float32, device=self.device)
        check_tensor("out", out, torch.float32, c.B * c.H * c.dv * c.dk, self.device)
        check_state(c, self.sizes, st, self.device)
        t = self._tensors(st)
        _lib.check(_lib.lib().qstate_dequantize(self._h, ctypes.byref(t), _ptr(out), self._stream(stream)),
                   "qstate_dequantize")
        return out

    def step(self, st: dict, q, k, v, decay, beta=None, out=None, step: int = 0, stream=None):
        """One decode step in place on `st`; returns o [B,H,dv] fp32."""
        import torch
        c = self.cfg
        if out is None:
            out = torch.empty((c.B, c.H, c.dv), dtype=torch.float32, device=self.device)
        check_inputs(c, c.B, self.device, q, k, v, decay, beta, out)
        check_state(c, self.sizes, st, self.device)
        t = self._tensors(st)
        inp = _lib.Inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta))
        _lib.check(_lib.lib().qstate_decode_step(self._h, ctypes.byref(t), ctypes.byref(inp), _ptr(out), step,
                                                 self._stream(stream)), "qstate_decode_step")
        return out

    def step_batch(self, pool: dict, slot, step, q, k, v, decay, beta=None, out=None, stream=None):
        """One decode step for n = len(slot) sequences whose states sit in the
        slots `slot` (int32 [n], device) of `pool` (this handle's B slots),
        each with its own step (uint64 stored as int64 [n], device); inputs
        [n,H,...]; returns o [n,H,dv] fp32."""
        import torch
        c = self.cfg
        n = int(slot.numel())
        if slot.dtype != torch.int32 or step.dtype not in (torch.int64, torch.uint64) or step.numel() != n:
            raise ValueError("slot must be int32 [n] and step 64-bit [n]")
        check_tensor("slot", slot, torch.int32, n, self.device)
        check_tensor("step", step, step.dtype, n, self.device)
        if out is None:
            out = torch.empty((n, c.H, c.dv), dtype=torch.float32, device=self.device)
        check_inputs(c, n, self.device, q, k, v, decay, beta, out)
        check_state(c, self.sizes, pool, self.device)
        t = self._tensors(pool)
        inp = _lib.Inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta))
        _lib.check(_lib.lib().qstate_decode_step_batch(self._h, ctypes.byref(t), ctypes.byref(inp), _ptr(out), n,
                                                       _ptr(slot), _ptr(step), self._stream(stream)),
                   "qstate_decode_step_batch")
        return out
