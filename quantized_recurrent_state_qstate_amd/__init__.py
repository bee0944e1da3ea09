"""qstate for MI355X: decode step of gated linear recurrences with a low-bit state.

The compute path is libqstate.so (hand-written gfx950 kernels behind the C
ABI in include/qstate.h); this package holds the kernels' sources, the
build step, a ctypes binding and the seeded workload generators.
Importing the package loads nothing; the library is loaded on first use.
"""
from .api import QState, StateConfig, build_map, plan  # noqa: F401

__all__ = ["QState", "StateConfig", "build_map", "plan"]
