"""The integer core of the 1-bit stage's scale folds on the CPU
(tests/sanitize/window_driver.cpp runs window_fold.hpp, the code the device
folds use): each workgroup's window sum through its carried 16-byte partial
and back, moved onto the final window with rounding to the nearest unit
(ties up), summed, and the test of whether the interval around the folded
integer can change its binary64 rounding -- all against exact Python
integers, whose conversion to float is correctly rounded.  No device code
runs here."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("window") / "window_driver")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-ffp-contract=off",
                    f"-I{ROOT}/include", f"-I{ROOT}/zero_partitioned_mixed_flatten_amd/csrc",
                    os.path.join(ROOT, "tests", "sanitize", "window_driver.cpp"), "-o", exe],
                   check=True, timeout=300, capture_output=True)
    return exe


def _moved(v, d):
    """v * 2^-d rounded to the nearest integer, ties up (d >= 0)."""
    return v if d == 0 else (v + (1 << (d - 1))) >> d


def _decides(w, half):
    """Whether every value within half/2 of w rounds to one binary64 (ends checked on the doubled values)."""
    return float(2 * w - half) == float(2 * w + half)


def _fold(driver, tmp_path, E, half, items):
    f = tmp_path / "fold.txt"
    lines = [f"{E} {half} {len(items)}"] + [f"{v >> 64} {v & ((1 << 64) - 1)} {e}" for v, e in items]
    f.write_text("\n".join(lines) + "\n")
    hi, lo, fits, dec, rt = subprocess.run([driver, "fold", str(f)], capture_output=True, text=True,
                                           check=True).stdout.split()
    return (int(hi) << 64) | int(lo), fits == "1", dec == "1", rt == "1"


@pytest.mark.parametrize("seed", range(12))
def test_fold_is_the_sum_of_rounded_moves(driver, tmp_path, seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(-149, 128))
    items = []
    for _ in range(int(rng.integers(1, 300))):
        v = (int(rng.integers(0, 1 << 30)) << 64) | int(rng.integers(0, 1 << 63)) * 2 + int(rng.integers(0, 2))
        gap = int(rng.choice([0, rng.integers(0, 8), rng.integers(0, 70), rng.integers(60, 300)]))
        items.append((v, E - gap))
    half = int(rng.integers(1, 1 << 41))
    w, fits, dec, rt = _fold(driver, tmp_path, E, half, items)
    want = sum(_moved(v, 2 * (E - e)) if 2 * (E - e) < 127 else 0 for v, e in items)
    assert rt and fits and w == want
    assert dec == _decides(w, half)


def test_moves_round_ties_up_and_drop_what_is_below_half_a_unit(driver, tmp_path):
    for d in (2, 4, 40, 64, 66, 124, 126):
        e = -(d // 2)
        for v, want in ((1 << (d - 1), 1), ((1 << (d - 1)) - 1, 0), (3 << (d - 1), 2), ((1 << d) + 1, 1)):
            if v >= 1 << 94:
                continue
            w, _, _, rt = _fold(driver, tmp_path, 0, 2, [(v, e)])
            assert rt and w == want, (d, v)
    for gap in (64, 127, 200, 276):                     # moves of 128 bits and more: below half a unit
        w, _, _, _ = _fold(driver, tmp_path, 127, 2, [((1 << 93) + 12345, 127 - gap), (5, 127)])
        assert w == 5


def test_interval_test_at_binary64_boundaries(driver, tmp_path):
    """W near a binary64 rounding boundary (ulp 2^28 at 2^80, ties halfway):
    the test says yes exactly when both ends of the interval round alike."""
    rng = np.random.default_rng(7)
    f = tmp_path / "dec.txt"
    cases = []
    for k in range(400):
        base = (1 << 80) + int(rng.integers(0, 1 << 40)) * (1 << 28)
        w = base + (1 << 27) + int(rng.integers(-3000, 3000))      # near a tie between two binary64
        half = int(rng.integers(1, 6000))
        cases.append((w, half))
    for scale in (80, 100, 121):                         # far from any boundary
        w = (1 << scale) + (1 << (scale - 60))
        cases.append((w, 1000))
    f.write_text("\n".join(f"{w >> 64} {w & ((1 << 64) - 1)} {h}" for w, h in cases) + "\n")
    got = subprocess.run([driver, "decides", str(f)], capture_output=True, text=True, check=True).stdout.split()
    assert len(got) == len(cases)
    want = [_decides(w, h) for w, h in cases]
    assert [g == "1" for g in got] == want
    assert 0 < sum(want) < len(want)                     # both outcomes occur
