"""Build libzero_mi355x.so (the C-ABI HIP library) in-tree for gfx950.

Flags that matter for the numerics:
  -ffp-contract=off                         no a*b+c -> fma contraction, so every
                                            operation rounds once, as specified;
  -fhip-fp32-correctly-rounded-divide-sqrt  IEEE division and square root;
  (default)                                 fp32/fp16 denormals are kept.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                            keep the compiler from forming packed
                                            fp32 arithmetic.
The host-only C++ sources are compiled by ROCm's clang++ as plain C++ (no
device pass), with the same no-contraction rule, and linked into the same
library.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzero_mi355x.so")
SOURCES = ["host.hip", "flatten.hip", "norm.hip", "adam.hip", "onebit.hip"]
HOST_SOURCES = ["host_step.cpp"]          # plain C++ (the CPU side of the offloaded step)
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


HOST_FLAGS = ["-x", "c++", "-std=c++17", "-O3", "-fPIC", "-ffp-contract=off", "-Wall",
              "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]


def host_cxx() -> str:
    for c in (os.environ.get("ZERO_HOST_CXX"), "/opt/rocm/llvm/bin/clang++"):
        if c and os.path.exists(c):
            return c
    return "clang++"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source into the in-tree shared library (always rebuilds)."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory() as objdir:
        objs = []
        for src in HOST_SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            cmd = [host_cxx(), *HOST_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}", "-o", tmp,
               *[os.path.join(CSRC, s) for s in SOURCES], "-x", "none", *objs, "-lpthread"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
