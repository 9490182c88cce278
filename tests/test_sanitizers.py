"""Sanitizer runs of the CPU code, on the CPU.

The oracle (C, with gcc) under AddressSanitizer + UndefinedBehaviorSanitizer,
and the host step (C++ with its AVX-512 kernels and worker pool, with ROCm's
clang++) under the same pair and, separately, under ThreadSanitizer.  The
drivers in tests/sanitize/ run every entry point on ragged sizes, misaligned
views and several worker counts with buffers sized exactly; a report from any
sanitizer aborts the driver (no recovery), which fails the test.  Device code
is not built here: only host compilers are used."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_flatten_amd", "csrc")
ROCM_CXX = "/opt/rocm/llvm/bin/clang++"
COMMON = ["-O1", "-g", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert r.stdout.strip().splitlines()[-1] in ("ok",) or r.stdout.startswith("skip"), r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=gnu11", *COMMON, "-fsanitize=address,undefined",
                    os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe], check=True, timeout=300)
    _run(exe)


@pytest.mark.skipif(not os.path.exists(ROCM_CXX) or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="ROCm clang++ / HIP runtime not available")
@pytest.mark.parametrize("sanitizer", ["address,undefined", "thread"])
def test_host_step_under_sanitizers(tmp_path, sanitizer):
    exe = str(tmp_path / "host_san")
    subprocess.run([ROCM_CXX, "-x", "c++", "-std=c++17", *COMMON, f"-fsanitize={sanitizer}",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}",
                    f"-I{CSRC}", os.path.join(CSRC, "host_step.cpp"), os.path.join(SAN, "host_step_driver.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-lpthread", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, timeout=600, capture_output=True)
    _run(exe)
