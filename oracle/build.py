"""Builds the CPU oracle (plain C, OpenMP) into oracle/liboracle.so.

The oracle is test infrastructure: building it is part of building the repository, but only
the tests, the smoke check and the benchmark's CPU-baseline leg load it.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off: every fused multiply-add in the canonical arithmetic is an explicit
# fmaf; no other multiply and add may be fused.  -mfma: fmaf compiles to the hardware
# instruction (checked at load time by oracle_cpu_ok).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-mfma",
          "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
