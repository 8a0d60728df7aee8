"""Builds the oracle's C sources into oracle/liboracle.so with gcc.

Test infrastructure only: the oracle is compiled so the checker exists; the
product library never links it.  Every binary32 step in the oracle must be a
single IEEE operation, so contraction and fast-math are off.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["codec.c", "ideal.c", "emulate.c", "threads.c"]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math", "-Wall", "-pthread", "-o", LIB + ".tmp"]
    cmd += [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
