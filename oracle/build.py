"""Compile the C oracle into ``oracle/liboracle.so`` (plain gcc, OpenMP).

Test infrastructure only: it builds the checker, it is never on the product
path.  ``-ffp-contract=off`` and no ``-ffast-math`` keep every fp32 operation
an individually rounded IEEE operation, which is what the oracle's readings
fix.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "convrot_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-std=c11", "-O3", "-fno-fast-math", "-ffp-contract=off",
    "-fno-finite-math-only", "-fopenmp", "-fPIC", "-shared", "-Wall",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
