"""Compile the C oracle into ``oracle/liboracle.so`` with gcc.

Test infrastructure: the oracle is built so that the tests, the smoke check
and the benchmark's CPU-baseline leg can call it; the product library never
links or loads it.  Flags keep the arithmetic as written: no fast-math, no
FMA contraction.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("q4k_oracle.c", "q5k_oracle.c", "q6k_oracle.c", "q3k_oracle.c", "w8a8_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle unconditionally and return the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *SRCS, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
