"""Builds the CPU oracle's shared library (oracle/libdwref.so) with gcc.

Test infrastructure only: the product library never links or loads it.
Built -O2 without -ffast-math, which would let the compiler reassociate the
fp64 sums and change what the oracle computes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dwref.c")
LIB = os.path.join(HERE, "libdwref.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-Werror", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Builds only when the library is missing or older than its source."""
    if (not os.path.exists(LIB)
            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
