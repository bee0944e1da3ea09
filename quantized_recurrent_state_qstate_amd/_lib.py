"""ctypes binding of libqstate.so (include/qstate.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
turns torch tensors into device pointers and torch streams into hipStream_t.
It raises if the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqstate.so")

ABI_VERSION = 2

QS_OK, QS_EINVAL, QS_EUNSUPPORTED, QS_ENOMEM, QS_EHIP = 0, -1, -2, -3, -4
KIND = {"additive": 0, "delta": 1}
DECAY = {"head": 0, "key": 1}
DTYPE = {"fp32": 0, "bf16": 1, "fp16": 2}
MAP = {"none": 0, "head": 1, "key": 2}
ROUNDING = {"nearest": 0, "stochastic": 1}
AXIS = {"value": 0, "key": 1, "head": 2}

EXPORTS = (
    "qstate_plan", "qstate_init", "qstate_quantize", "qstate_decode_step", "qstate_decode_step_batch",
    "qstate_dequantize", "qstate_build_map", "qstate_destroy", "qstate_strerror",
    "qstate_last_error", "qstate_kernel_name",
)


class Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("kind", ctypes.c_int32), ("decay_mode", ctypes.c_int32),
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("qbits", ctypes.c_int32), ("hp_dtype", ctypes.c_int32), ("map_mode", ctypes.c_int32),
        ("map", ctypes.POINTER(ctypes.c_uint8)), ("in_dtype", ctypes.c_int32),
        ("rounding", ctypes.c_int32), ("sr_bits", ctypes.c_int32),
        ("bdr", ctypes.c_int32), ("bdr_bound", ctypes.c_float),
        ("lrb_rank", ctypes.c_int32), ("lrb_period", ctypes.c_int32), ("lrb_theta", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("scale_dtype", ctypes.c_int32), ("lrb_dtype", ctypes.c_int32),
        ("scale_axis", ctypes.c_int32),
    ]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("codes", "scales", "hp", "lrb_W", "lrb_U", "lrb_n")]


class Tensors(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("hp", ctypes.c_void_p),
                ("lrb_W", ctypes.c_void_p), ("lrb_U", ctypes.c_void_p), ("lrb_n", ctypes.c_void_p)]


class Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("decay", ctypes.c_void_p), ("beta", ctypes.c_void_p)]


class QStateError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libqstate.so (built in-tree by build()); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libqstate.so not found at {LIB_PATH}; build it with "
                "`python -m quantized_recurrent_state_qstate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.qstate_plan.argtypes = [P(Config), P(Sizes)]
        L.qstate_init.argtypes = [P(Config), P(vp), P(Sizes)]
        L.qstate_quantize.argtypes = [vp, vp, P(Tensors), ctypes.c_uint64, vp]
        L.qstate_decode_step.argtypes = [vp, P(Tensors), P(Inputs), vp, ctypes.c_uint64, vp]
        L.qstate_decode_step_batch.argtypes = [vp, P(Tensors), P(Inputs), vp, ctypes.c_int32, vp, vp, vp]
        L.qstate_dequantize.argtypes = [vp, P(Tensors), vp, vp]
        L.qstate_build_map.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, vp]
        for f in ("qstate_plan", "qstate_init", "qstate_quantize", "qstate_decode_step",
                  "qstate_decode_step_batch", "qstate_dequantize", "qstate_build_map"):
            getattr(L, f).restype = ctypes.c_int
        L.qstate_destroy.argtypes = [vp]
        L.qstate_destroy.restype = None
        L.qstate_strerror.argtypes = [ctypes.c_int]
        L.qstate_strerror.restype = ctypes.c_char_p
        L.qstate_last_error.argtypes = []
        L.qstate_last_error.restype = ctypes.c_char_p
        L.qstate_kernel_name.argtypes = [vp]
        L.qstate_kernel_name.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def check(status: int, where: str) -> None:
    if status != QS_OK:
        L = lib()
        detail = L.qstate_last_error().decode() or L.qstate_strerror(status).decode()
        raise QStateError(status, where, detail)
