"""Pins for the oracle's squared-L2-norm + inf/NaN reduction.

The oracle claims the sum of squares is exact and rounded once to binary64.
That is checked against exact rational sums (fractions.Fraction, whose float()
is correctly rounded) on small vectors and against math.fsum (a correctly
rounded sum) on larger ones, including mixes of the largest and the smallest
binary16 magnitudes where a plain binary64 running sum would lose bits."""
import math
from fractions import Fraction

import numpy as np
import pytest


def _finite_f16(rng, n, lo_exp=0, hi_exp=30):
    e = rng.integers(lo_exp, hi_exp + 1, n).astype(np.uint16)
    f = rng.integers(0, 1024, n).astype(np.uint16)
    s = rng.integers(0, 2, n).astype(np.uint16)
    return (s << 15) | (e << 10) | f


def _squares64(h):
    x = h.view(np.float16).astype(np.float64)
    return x * x                                   # exact: 22-bit significands


@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_sum_small(oracle, seed):
    rng = np.random.default_rng(seed)
    h = _finite_f16(rng, int(rng.integers(1, 300)))
    exact = sum((Fraction(float(x)) ** 2 for x in h.view(np.float16).astype(np.float64)), Fraction(0))
    s, ovf = oracle.norm_overflow(h)
    assert ovf == 0
    assert s == float(exact)                       # float(Fraction) rounds correctly


@pytest.mark.parametrize("seed", range(3))
def test_fsum_large(oracle, seed):
    rng = np.random.default_rng(100 + seed)
    h = _finite_f16(rng, 200_000)
    s, ovf = oracle.norm_overflow(h)
    assert ovf == 0 and s == math.fsum(_squares64(h))


def test_extreme_magnitude_mix_is_exact(oracle):
    # One 65504 and 2^20 smallest subnormals: 65504^2 + 2^20 * 2^-48.  A
    # binary64 running sum drops every tiny term; the exact sum keeps them.
    h = np.full((1 << 20) + 1, 0x0001, np.uint16)
    h[0] = 0x7BFF
    s, ovf = oracle.norm_overflow(h)
    exact = Fraction(65504) ** 2 + Fraction(1 << 20, 1 << 48)
    assert ovf == 0 and s == float(exact)
    naive = 0.0
    for v in _squares64(h[:1000]):
        naive += v
    assert naive == 65504.0 ** 2                   # shows the naive sum losing them


def test_subnormals_only(oracle):
    h = np.arange(1, 1024, dtype=np.uint16)        # every positive subnormal
    s, _ = oracle.norm_overflow(h)
    exact = sum(Fraction(k, 1 << 24) ** 2 for k in range(1, 1024))
    assert s == float(exact)


def test_sign_does_not_matter(oracle):
    rng = np.random.default_rng(7)
    h = _finite_f16(rng, 5000)
    assert oracle.norm_overflow(h)[0] == oracle.norm_overflow(h ^ np.uint16(0x8000))[0]


def test_every_inf_and_nan_pattern_flags(oracle):
    rng = np.random.default_rng(8)
    base = _finite_f16(rng, 64)
    specials = np.array([(s << 15) | (31 << 10) | f for s in (0, 1) for f in range(1024)], np.uint16)
    for sp in specials:
        h = base.copy()
        h[int(rng.integers(64))] = sp
        s, ovf = oracle.norm_overflow(h)
        assert ovf == 1 and s == math.inf
    s, ovf = oracle.norm_overflow(base)
    assert ovf == 0 and math.isfinite(s)


def test_largest_finite_is_not_overflow(oracle):
    h = np.array([0x7BFF, 0xFBFF], np.uint16)      # +-65504
    s, ovf = oracle.norm_overflow(h)
    assert ovf == 0 and s == 2 * 65504.0 ** 2


def test_empty_and_zeros(oracle):
    assert oracle.norm_overflow(np.zeros(0, np.uint16)) == (0.0, 0)
    assert oracle.norm_overflow(np.array([0x0000, 0x8000], np.uint16)) == (0.0, 0)
