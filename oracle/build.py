"""Compile the C oracle into ``oracle/liboracle.so`` with gcc.

Test infrastructure: the oracle is built so that the tests, the smoke check
and the benchmark's CPU-baseline leg can call it; the product library never
links or loads it.  Flags keep the arithmetic as written: no fast-math, no
FMA contraction.

``liboracle_omp.so`` is the same source built with OpenMP: its row loops run
on all host cores (one whole output row per thread, summed in the same
order), for the benchmark's all-cores CPU-baseline leg only.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("q4k_oracle.c", "q5k_oracle.c", "q6k_oracle.c", "q3k_oracle.c", "w8a8_oracle.c")]
LIB = os.path.join(HERE, "liboracle.so")
LIB_OMP = os.path.join(HERE, "liboracle_omp.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unknown-pragmas"]


def _compile(out: str, extra, verbose: bool) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, *SRCS, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile both oracle builds unconditionally; returns the plain library's path."""
    _compile(LIB, [], verbose)
    _compile(LIB_OMP, ["-fopenmp"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
