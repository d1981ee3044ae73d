"""Compile the fp64 attention oracle (plain C + OpenMP) into oracle/liboracle.so.

Test infrastructure: the library built here is only loaded by the test suite,
the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # x86-64-v3 (AVX2 + FMA) runs on every host CPU this targets; -ffp-contract=off keeps
    # each multiply and add a separately rounded fp64 operation, as written.
    cmd = ["gcc", "-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
