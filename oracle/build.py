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
# AddressSanitizer + UndefinedBehaviorSanitizer build for checking the oracle
# itself: clang from the ROCm toolchain, so that it shares one sanitizer
# runtime with the sanitized HIP host code in the same process (load it with
# FP8A_ORACLE_LIB=<path> and the runtime preloaded)
SAN_LIB = os.path.join(HERE, "liboracle_san.so")
SAN_CC = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
             "-shared-libasan"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    cmd = [SAN_CC if sanitize else "gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-frounding-math", "-Wall", "-pthread", "-o", out + ".tmp"]
    if sanitize:
        cmd += SAN_FLAGS
    cmd += [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
