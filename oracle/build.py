"""Build step for the CPU oracle library (test infrastructure only).

Compiles oracle.c with gcc into oracle/liboracle.so: IEEE binary32 with no
FMA contraction and no fast-math, OpenMP over independent rows.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    """Compile the oracle library and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
