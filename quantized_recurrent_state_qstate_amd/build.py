"""Build libqstate.so (gfx950) in-tree with hipcc.

Flags:
  --offload-arch=gfx950            CDNA4 code object only
  -ffp-contract=off                only the explicit fmaf() calls fuse, so the
                                   fp32 operation sequence is the one written
  -fno-gpu-flush-denormals-to-zero fp32 subnormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                   no packed fp32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqstate.so")
SOURCES = [os.path.join(CSRC, "qstate_kernels.hip"), os.path.join(CSRC, "qstate_host.cpp")]
HEADERS = [os.path.join(CSRC, "qstate_internal.hpp"), os.path.join(CSRC, "qstate_device.hpp"),
           os.path.join(INCLUDE, "qstate.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libqstate.so; returns its path."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
