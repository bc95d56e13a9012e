"""Build the CPU oracle library (test infrastructure only).

Compiles ``oracle_gemm.c`` with gcc into ``liboracle.so`` beside it.  The flags
keep IEEE semantics: no FMA contraction, no fast-math, SSE2 doubles.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-Wall", "-Wextra"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
