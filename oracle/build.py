"""Build the oracle's shared library with gcc.

Test infrastructure: the oracle is only for the test suite, the smoke check
and the benchmark's CPU-baseline leg.

The flags keep every floating-point operator a single IEEE-754
round-to-nearest-even operation: no contraction into fused multiply-adds, no
fast-math, SSE arithmetic (x86-64 default, no x87 excess precision).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zero_oracle.c")
LIB = os.path.join(HERE, "liboracle_zero.so")

CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-unsafe-math-optimizations", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile zero_oracle.c into liboracle_zero.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only when the library is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
