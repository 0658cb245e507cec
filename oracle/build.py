"""Compile the fp64 oracle (plain C, gcc, OpenMP) into oracle/libefla_oracle.so.

Test infrastructure: the library it builds is loaded only by the tests, the
smoke check and the CPU-baseline leg of the benchmark.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "efla_oracle.c")
LIB = os.path.join(HERE, "libefla_oracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without -ffast-math: IEEE fp64 semantics, no reassociation.
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
