"""Build step for the CPU oracle library (test infrastructure only).

Compiles oracle.c with gcc into oracle/liboracle.so: IEEE binary32 with no
FMA contraction and no fast-math, OpenMP over independent rows.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


# Host sanitizers for the checker itself: AddressSanitizer (out-of-bounds and
# use-after-free on the host arrays) and UndefinedBehaviorSanitizer (signed
# overflow, bad shifts, misaligned loads), every finding fatal.
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile the oracle library and return its path (with sanitize, an
    instrumented build at `out`, which a process must load after preloading
    the AddressSanitizer runtime)."""
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
