"""Build libzero_mi355x.so (the C-ABI HIP library) in-tree for gfx950.

Flags that matter for the numerics:
  -ffp-contract=off                         no a*b+c -> fma contraction, so every
                                            operation rounds once, as specified;
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE division and square root;
  (default)                                 fp32/fp16 denormals are kept.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                            keep the compiler from forming packed
                                            fp32 arithmetic.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzero_mi355x.so")
SOURCES = ["host.hip", "flatten.hip", "norm.hip", "adam.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into the in-tree shared library (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
