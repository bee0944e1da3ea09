"""Build libqstate.so (gfx950) in-tree with hipcc.

Translation units:
  qstate_step_<family>.hip   one per step-kernel family (dense, mixed, keymap,
                             lrb, grouped), compiled once per (qbits, rounding)
                             pair with -DQS_QB=<8|4> -DQS_RND=<0|1|2> (lrb once
                             per kind too, -DQS_DELTA=<0|1>; keymap once per
                             dk, -DQS_DK=<64|128|256>): 48 objects that
                             compile in parallel
  qstate_misc.hip            quantize / dequantize / fill kernels, dispatch
  qstate_host.cpp            the C ABI: validation, planning, launches
Objects go to build/qstate/ and link into
quantized_recurrent_state_qstate_amd/libqstate.so.  build(force=False)
recompiles only objects older than their source or any header it includes
(followed through the local #include "..." lines).

Flags:
  --offload-arch=gfx950            CDNA4 code object only
  -ffp-contract=off                only the explicit fmaf() calls fuse, so the
                                   fp32 operation sequence is the one written
  -fno-gpu-flush-denormals-to-zero fp32 subnormals are kept
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                   no packed fp32 VALU instructions
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "build", "qstate")
LIB = os.path.join(PKG, "libqstate.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]

FAMILIES = ("dense", "mixed", "keymap", "lrb", "grouped")
QR = [(qb, rnd) for qb in (8, 4) for rnd in (0, 1, 2)]
RND_NAME = {0: "rtn", 1: "sr16", 2: "sr8"}


def units():
    """(source, extra flags, object path) of every translation unit."""
    out = []
    for fam in FAMILIES:
        src = os.path.join(CSRC, f"qstate_step_{fam}.hip")
        for qb, rnd in QR:
            if fam == "lrb":   # the longest units: one per kind as well
                for delta in (0, 1):
                    obj = os.path.join(OBJ, f"qstate_step_{fam}_q{qb}_{RND_NAME[rnd]}_d{delta}.o")
                    out.append((src, [f"-DQS_QB={qb}", f"-DQS_RND={rnd}", f"-DQS_DELTA={delta}"], obj))
                continue
            if fam == "keymap":   # one per dk as well
                for dk in (64, 128, 256):
                    obj = os.path.join(OBJ, f"qstate_step_{fam}_q{qb}_{RND_NAME[rnd]}_k{dk}.o")
                    out.append((src, [f"-DQS_QB={qb}", f"-DQS_RND={rnd}", f"-DQS_DK={dk}"], obj))
                continue
            obj = os.path.join(OBJ, f"qstate_step_{fam}_q{qb}_{RND_NAME[rnd]}.o")
            out.append((src, [f"-DQS_QB={qb}", f"-DQS_RND={rnd}"], obj))
    for name in ("qstate_misc.hip", "qstate_host.cpp"):
        out.append((os.path.join(CSRC, name), [], os.path.join(OBJ, name + ".o")))
    return out


_INC = re.compile(r'^\s*#\s*include\s+"([^"]+)"', re.M)


def deps(src: str) -> set:
    """The source and every local header it includes, transitively."""
    seen, todo = set(), [src]
    while todo:
        p = todo.pop()
        if p in seen or not os.path.exists(p):
            continue
        seen.add(p)
        with open(p) as f:
            for name in _INC.findall(f.read()):
                for d in (os.path.dirname(p), CSRC, INCLUDE):
                    q = os.path.join(d, name)
                    if os.path.exists(q):
                        todo.append(q)
                        break
    return seen


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in deps(src))


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(_stale(s, o) or os.path.getmtime(o) > t for s, _, o in units())


def _compile(unit, verbose: bool) -> str:
    src, extra, obj = unit
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(extra)}:\n{r.stderr}")
    return obj


def build(force: bool = True, verbose: bool = False, jobs: int = 0) -> str:
    """Compile libqstate.so (every unit when force, else the stale ones); returns its path."""
    if not force and not stale():
        return LIB
    os.makedirs(OBJ, exist_ok=True)
    todo = [u for u in units() if force or _stale(u[0], u[2])]
    jobs = jobs or min(16, os.cpu_count() or 1)
    # the longest units first: low-rank bypass, then the other step kernels
    todo.sort(key=lambda u: 0 if ("qstate_step_lrb" in u[0] or "_k256" in u[2]) else (1 if "qstate_step_" in u[0] else 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda u: _compile(u, verbose), todo))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, _, o in units()], "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv or "-f" in sys.argv, verbose="-v" in sys.argv))
