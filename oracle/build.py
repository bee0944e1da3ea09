"""Build the CPU oracle (test infrastructure only).

Compiles ``qs_oracle.c`` with gcc into ``liboracle.so`` next to this file.
Flags: ``-ffp-contract=off`` so that only the explicit ``fmaf`` calls fuse,
no fast-math, so IEEE division, rounding and subnormals hold.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qs_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle; returns the path of the shared library."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(
        os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "qs_oracle.h"))
    ):
        return LIB
    tmp = LIB + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
        "-fno-fast-math", "-shared", "-fPIC", SRC, "-o", tmp, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
