"""The exact norm's integer limbs on the CPU: a workgroup's sum packed into its
16-byte partial (make_partial, with the carry), partials folded as the decide
kernels fold them (fold_partial: four signed 64-bit limbs, no carry-out used),
and the total turned into 128 bits (limbs_to_u128) -- the same
exact_norm.hpp functions the device runs (tests/sanitize/window_driver.cpp),
against Python integers.  This is the arithmetic that carries every exact sum
across workgroups; the bound it relies on (up to 2^30 partials below 2^126
fold without a carry out of any limb) is exercised at its limit."""
import numpy as np
import pytest

from test_window_host import driver  # noqa: F401  (the built driver, shared)
import subprocess


def _fold(driver, tmp_path, rows):
    f = tmp_path / "limbs.txt"
    f.write_text("\n".join(f"{v >> 64} {v & ((1 << 64) - 1)} {st} {rep}" for v, st, rep in rows) + "\n")
    hi, lo, fits, flag = subprocess.run([driver, "limbs", str(f)], capture_output=True, text=True,
                                        check=True).stdout.split()
    return (int(hi) << 64) | int(lo), fits == "1", int(flag)


@pytest.mark.parametrize("seed", range(8))
def test_partials_fold_to_their_exact_sum(driver, tmp_path, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(int(rng.integers(1, 2000))):
        bits = int(rng.integers(1, 127))
        v = int.from_bytes(rng.bytes(16), "little") >> (128 - bits)      # below 2^126
        rows.append((v, int(rng.integers(0, 4)) if rng.integers(0, 50) == 0 else 0, int(rng.integers(1, 4))))
    total, fits, flag = _fold(driver, tmp_path, rows)
    want = sum(v * rep for v, _, rep in rows)
    want_flag = 0
    for _, st, _ in rows:
        want_flag |= st
    assert fits == (want < 1 << 128) and flag == want_flag
    if fits:
        assert total == want


def test_limb_edges(driver, tmp_path):
    """All-ones limbs, a value one below the partial bound, single limbs, and
    2^30 copies of the largest partial (the fold's stated limit): the total is
    exact while it stays below 2^128 and reported as not fitting above."""
    top = (1 << 126) - 1
    cases = [[(top, 0, 1)], [((1 << 96) - 1, 0, 5)], [(1 << 95, 0, 3), ((1 << 64) - 1, 0, 7)],
             [(0xFFFFFFFF, 0, 1 << 20)], [(1 << 125, 0, 3)], [(top, 0, 4)]]
    for rows in cases:
        total, fits, flag = _fold(driver, tmp_path, rows)
        want = sum(v * rep for v, _, rep in rows)
        assert flag == 0 and fits == (want < 1 << 128), rows
        if fits:
            assert total == want, rows
    total, fits, _ = _fold(driver, tmp_path, [((1 << 97) - 1, 0, 1 << 30)])     # 2^30 partials just below 2^97
    assert fits and total == ((1 << 97) - 1) << 30


def test_status_bits_travel_with_the_partial(driver, tmp_path):
    for st in (1, 2, 3):
        total, _, flag = _fold(driver, tmp_path, [(12345, 0, 2), (1 << 100, st, 1)])
        assert flag == st and total == 2 * 12345 + (1 << 100)
