"""The wide exact sum's integer arithmetic on the CPU (tests/sanitize/wide_driver.cpp
runs the same square decomposition, carry, rounding and 2^-48-unit extraction
that the device pass in wide_sum.hpp uses), against exact Python arithmetic:
integers built from the IEEE-754 fields of every value, math.fsum, and
float(Fraction), whose rounding is correct.  No device code runs here."""
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
F32_MAX = float(np.finfo(np.float32).max)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("wide") / "wide_driver")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-ffp-contract=off",
                    f"-I{ROOT}/include", f"-I{ROOT}/zero_partitioned_mixed_flatten_amd/csrc",
                    os.path.join(ROOT, "tests", "sanitize", "wide_driver.cpp"), "-o", exe],
                   check=True, timeout=300, capture_output=True)
    return exe


def _exact_units298(x):
    """sum of x^2 in units of 2^-298, from the binary32 fields (x = M * 2^e)."""
    total = 0
    for b in (x.view(np.uint32) & np.uint32(0x7FFFFFFF)).tolist():
        field, m = b >> 23, b & 0x7FFFFF
        if field:
            m |= 1 << 23
        e = field - 150 if field else -149
        total += (m * m) << (2 * e + 298)
    return total


def _sum(driver, x, tmp_path):
    f = tmp_path / "x.bin"
    np.ascontiguousarray(x, dtype=np.float32).tofile(f)
    out = subprocess.run([driver, "sum", str(f)], capture_output=True, text=True, check=True).stdout.split()
    return float.fromhex(out[0]), out[1] == "1", (int(out[2]) << 64) | int(out[3])


def _values(rng, n, lo, hi):
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    x = np.minimum(mant * np.exp2(rng.integers(lo, hi + 1, n) - 23.0), F32_MAX).astype(np.float32)
    return x * np.where(rng.integers(0, 2, n) == 1, -1, 1).astype(np.float32)


@pytest.mark.parametrize("seed,lo,hi", [(0, -149, 127), (1, -149, -120), (2, -30, 30), (3, 100, 127),
                                        (4, -24, 15), (5, -149, 127)])
def test_sum_of_squares_is_exact_and_rounded_once(driver, tmp_path, seed, lo, hi):
    rng = np.random.default_rng(seed)
    x = _values(rng, int(rng.integers(1, 3000)), lo, hi)
    if seed == 4:                                   # binary16 values: whole numbers of 2^-48 units
        x = x.astype(np.float16).astype(np.float32)
    if seed == 5:
        x[rng.integers(0, x.size, x.size // 2)] = 0.0
    s, whole, units = _sum(driver, x, tmp_path)
    exact = _exact_units298(x)
    assert s == float(Fraction(exact, 1 << 298)) == math.fsum(x.astype(np.float64) ** 2)
    if exact % (1 << 250) == 0 and exact >> 250 < (1 << 128):
        assert whole and units == exact >> 250
    else:
        assert not whole


def test_named_cases(driver, tmp_path):
    # a binary64 tie broken only by a square 2^-120 below the largest; the tie without it; the extremes
    assert _sum(driver, np.array([1.0, 2.0 ** -27, -(2.0 ** -27), 2.0 ** -60], np.float32), tmp_path)[0] == \
        1.0 + 2.0 ** -52
    assert _sum(driver, np.array([1.0, 2.0 ** -27, -(2.0 ** -27)], np.float32), tmp_path)[0] == 1.0
    assert _sum(driver, np.array([2.0 ** -149], np.float32), tmp_path)[0] == 2.0 ** -298
    top = np.full(1000, F32_MAX, np.float32)
    assert _sum(driver, top, tmp_path)[0] == float(Fraction(int(F32_MAX)) ** 2 * 1000)
    assert _sum(driver, np.zeros(5, np.float32), tmp_path)[:2] == (0.0, True)


def test_rounding_of_arbitrary_digit_strings(driver, tmp_path):
    """to_f64 on carried 20-digit integers of every length, with and without
    bits below the rounding point, against float(Fraction)."""
    rng = np.random.default_rng(9)
    recs, refs = [], []
    for t in range(20):
        for _ in range(40):
            d = np.zeros(20, np.uint64)
            d[:t + 1] = rng.integers(0, 1 << 32, t + 1, dtype=np.uint64)
            if t and rng.integers(0, 2):
                d[:max(0, t - 2)] = 0                # exact below the top three digits
            if t >= 2 and rng.integers(0, 4) == 0:   # a tie: 53 kept bits, then exactly one half
                top = 32 * t + int(rng.integers(0, 32))
                sig = int(rng.integers(1 << 52, 1 << 53))
                v = (sig << (top - 52)) | (1 << (top - 53))
                d = np.array([(v >> (32 * k)) & 0xFFFFFFFF for k in range(20)], np.uint64)
            if not d.any():
                d[0] = 1
            recs.append(d)
            refs.append(float(Fraction(sum(int(x) << (32 * k) for k, x in enumerate(d)), 1 << 298)))
    f = tmp_path / "d.bin"
    np.stack(recs).astype(np.uint64).tofile(f)
    out = subprocess.run([driver, "digits", str(f)], capture_output=True, text=True, check=True).stdout.split()
    assert [float.fromhex(o) for o in out] == refs
