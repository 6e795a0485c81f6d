"""Compile the float64 oracle (oracle.c) into liboracle.so with the host C compiler.

Test infrastructure: the oracle is built next to its source and loaded only by
the tests, the smoke check and the benchmark's CPU-baseline leg. Plain -O2, no
fast-math, so IEEE semantics (infinities, NaN, exact integer sums) hold.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra=None, cc: str = "gcc") -> str:
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp"
    cmd = [cc, *CFLAGS, *(extra or []), src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
