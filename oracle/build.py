"""Build the CPU oracle's shared library (plain C, gcc, OpenMP).

Test infrastructure: the library this builds is loaded only by the test
suite, the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

# -ffp-contract=off: every product and sum is rounded as written, so the
# per-token loop and the round executor produce identical bits.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
