"""Builds the C oracle into oracle/_liboracle.so with the host C compiler.

Test infrastructure: the oracle is the CPU reference the HIP library is checked
against.  Building it is allowed everywhere; only tests, the smoke check and the
benchmark's CPU baseline leg load it.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv_verify_oracle.c")
LIB = os.path.join(HERE, "_liboracle.so")

# -ffp-contract=off: no mul+add is fused behind the source's back; the only fused
# multiply-adds are the explicit fmaf() calls of the conv.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra"]


def build(src: str = SRC, lib: str = LIB, cc: str = "gcc", quiet: bool = False) -> str:
    cmd = [cc, *CFLAGS, src, "-o", lib + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(lib + ".tmp", lib)
    if not quiet and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    return lib


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build(quiet=True)
    return LIB


if __name__ == "__main__":
    print(build())
