"""Compile the CPU oracle (test infrastructure) into oracle/libmta_oracle.so.

The flags matter for what the oracle means: no contraction into fused
multiply-add, no fast-math, so each float32 operation of the pages' formulas
is rounded on its own.  x86-64's baseline target has no FMA unit in use and
computes float in SSE registers (no x87 excess precision).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mta_oracle.c")
LIB = os.path.join(HERE, "libmta_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-unsafe-math-optimizations", "-Wall",
          "-Wextra"]


def build(verbose=False):
    """Compile the oracle; always recompiles.  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
