"""Compile the reference oracle (test infrastructure) into oracle/liboracle_qr.so with gcc.

Only the tests, the smoke check and the benchmark's CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qr_oracle.c")
LIB = os.path.join(HERE, "liboracle_qr.so")


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the library path."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
           "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
