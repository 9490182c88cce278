"""Pins for the oracle's 1-bit Adam compression stage (Tang et al. 2021,
Algorithm 1: frozen variance, scaled-sign momentum compression with worker and
server error feedback; one data-parallel rank is its own server).

The scale s = ||x||_2/sqrt(d) comes from the exact sum of squares rounded once
to binary64; the sum is checked against exact rational arithmetic
(fractions.Fraction, whose float() rounds correctly) and math.fsum, and s
against closed forms (equal magnitudes, one nonzero element, powers of two)
and its norm-preserving property.  The sign bits are checked against numpy's
packbits.  The step is checked against closed forms of the algorithm
(equal-magnitude momentum compresses without error, error feedback
telescopes, the variance stays frozen) rather than a retyped copy of it."""
import math
from fractions import Fraction

import numpy as np
import pytest

import shardgen

LR, B1, EPS, WD = 1e-4, 0.9, 1e-8, 0.01


def _exact_sum(x):
    """The sum of squares as an exact rational, rounded once by float()."""
    return float(sum((Fraction(float(v)) ** 2 for v in x.astype(np.float64)), Fraction(0)))


@pytest.mark.parametrize("seed", range(6))
def test_scale_sum_matches_exact_rationals(oracle, seed):
    # magnitudes spread over 40 binades starting anywhere from 2^-140
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 500))
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    lo = int(rng.integers(-140, -10))
    x = (mant * np.exp2(rng.integers(lo, lo + 40, n).astype(np.float64))).astype(np.float32)
    x *= np.where(rng.integers(0, 2, n) == 1, -1, 1).astype(np.float32)
    s, S = oracle.onebit_scale(x)
    assert S == _exact_sum(x)
    assert S == math.fsum(x.astype(np.float64) ** 2)
    assert s == np.float32(math.sqrt(S / n))        # correctly rounded binary64 division and root


def test_scale_keeps_squares_far_below_the_largest(oracle):
    # 1 + 2 * 2^-54 lies exactly halfway between 1 and 1 + 2^-52, so the
    # 2^-120 from 2^-60 decides the rounding of the sum (upward); without it
    # the tie goes to even.
    x = np.array([1.0, 2.0 ** -27, -(2.0 ** -27), 2.0 ** -60], np.float32)
    assert oracle.onebit_scale(x)[1] == 1.0 + 2.0 ** -52
    assert oracle.onebit_scale(x[:3])[1] == 1.0
    y = np.array([2.0 ** 100, 2.0 ** -149], np.float32)              # 2^200 + 2^-298: rounds to 2^200
    assert oracle.onebit_scale(y)[1] == 2.0 ** 200


def test_scale_closed_forms(oracle):
    for a in (1.0, 2.0 ** -30, 3.5, 1e-20, 6e4):
        x = np.array([a, -a, a, a, -a, -a, a, a], np.float32)
        assert oracle.onebit_scale(x)[0] == np.float32(a)          # equal magnitudes: s = |x|
    x = np.zeros(16, np.float32)
    x[5] = -8.0
    assert oracle.onebit_scale(x)[0] == 2.0                         # one nonzero of 16: 8/sqrt(16)
    assert oracle.onebit_scale(np.zeros(7, np.float32)) == (0.0, 0.0)
    assert oracle.onebit_scale(np.zeros(0, np.float32)) == (0.0, 0.0)


@pytest.mark.parametrize("special", [[np.inf], [-np.inf], [np.nan], [np.inf, np.nan], [-np.inf, 3e38]])
def test_scale_of_non_finite_vectors(oracle, special):
    """A vector holding an inf or a NaN (only binary32 overflow in the stage's
    own adds can put one there): the sum of squares is what IEEE arithmetic
    over the squares gives -- math.fsum of the Python squares: +inf, or NaN
    with any NaN -- and the scale fp32(sqrt(S/d)) follows."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1000) * 1e3).astype(np.float32)
    x[rng.choice(1000, len(special), replace=False)] = np.array(special, np.float32)
    s, S = oracle.onebit_scale(x)
    ref = math.fsum(float(v) * float(v) for v in x)
    assert (math.isnan(S) and math.isnan(ref)) or S == ref == math.inf
    want = np.float32(math.sqrt(ref / x.size))
    assert (np.isnan(s) and np.isnan(want)) or s == want == np.inf


@pytest.mark.parametrize("seed", range(3))
def test_scale_preserves_the_norm(oracle, seed):
    rng = np.random.default_rng(10 + seed)
    x = (rng.standard_normal(100_000) * 1e-3).astype(np.float32)
    s, _ = oracle.onebit_scale(x)
    norm = math.sqrt(math.fsum(x.astype(np.float64) ** 2))
    assert s * math.sqrt(x.size) == pytest.approx(norm, rel=1e-7)


def test_pack_is_numpy_packbits(oracle):
    rng = np.random.default_rng(3)
    for n in (1, 7, 8, 9, 1001):
        x = rng.standard_normal(n).astype(np.float32)
        x[::5] = 0.0
        x[1::7] = -0.0
        ref = np.packbits(~np.signbit(x) | (x == 0), bitorder="little")
        assert np.array_equal(oracle.onebit_pack(x), ref)


def _arrays(seed, n, v_scale=1e-6):
    rng = np.random.default_rng(seed)
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v32 = (np.abs(rng.standard_normal(n)) * v_scale).astype(np.float32)
    return (shardgen.to_f16_bits(p32), p32, np.zeros(n, np.float32), v32, np.zeros(n, np.float32),
            np.zeros(n, np.float32))


def _decided(oracle, S, g16):
    st = oracle.new_state(S)
    s, o = oracle.norm_overflow(g16)
    oracle.decide(st, oracle.hparams(lr=LR, max_grad_norm=0.0), s, o)
    return st


def test_equal_magnitudes_compress_without_error(oracle):
    # g = +-a with a power of two: m = (1-b1) g has one magnitude, so both
    # compressions are exact (s = |m|), both errors stay 0 and the momentum is
    # the plain one; the update is then closed form.
    n, S, a = 4096, 2.0 ** 10, 2.0 ** -6
    rng = np.random.default_rng(4)
    signs = np.where(rng.integers(0, 2, n) == 1, 1.0, -1.0).astype(np.float32)
    g16 = shardgen.to_f16_bits(signs * np.float32(a * S))
    p16, p32, m32, v32, ew, es = _arrays(5, n)
    p0, v0 = p32.astype(np.float64), v32.copy()
    st = _decided(oracle, S, g16)
    bw, bs, (sw, ss) = oracle.onebit_step(st, p16, p32, m32, v32, ew, es, g16)
    m_ref = np.float32(st.omb1) * (signs * np.float32(a))
    assert sw == ss == abs(float(m_ref[0]))
    assert not ew.any() and not es.any()
    assert m32.tobytes() == m_ref.tobytes()
    assert np.array_equal(bw, np.packbits(signs > 0, bitorder="little")) and np.array_equal(bw, bs)
    upd = m_ref.astype(np.float64) / (np.sqrt(v0.astype(np.float64)) + EPS) + WD * p0
    ref = p0 - LR * upd
    assert np.all(np.abs(p32 - ref) <= 1e-6 * np.maximum(np.abs(ref), np.abs(p0)))
    assert v32.tobytes() == v0.tobytes()                            # the variance is frozen
    assert np.array_equal(p16, shardgen.to_f16_bits(p32))


def test_error_feedback_telescopes(oracle):
    """Over T steps the worker's compressed outputs sum to the momenta plus the
    initial error minus the final error; the server's outputs sum to the
    worker outputs plus its own error change (exact in real arithmetic; here
    within the fp32 roundings of the error updates)."""
    n, T, S = 20_000, 12, 2.0 ** 12
    p16, p32, m32, v32, ew, es = _arrays(6, n)
    rng = np.random.default_rng(7)
    sum_m = np.zeros(n)
    sum_cw = np.zeros(n)
    sum_cs = np.zeros(n)
    st = oracle.new_state(S)
    hp = oracle.hparams(lr=LR, max_grad_norm=0.0)
    for _ in range(T):
        g16 = shardgen.to_f16_bits((rng.standard_normal(n) * 1e-3 * S).astype(np.float32))
        s, o = oracle.norm_overflow(g16)
        oracle.decide(st, hp, s, o)
        g = g16.view(np.float16).astype(np.float64) * float(np.float32(st.gmul))
        m_local = np.float64(st.beta1) * m32.astype(np.float64) + np.float64(st.omb1) * g   # before the step
        bw, bs, (sw, ss) = oracle.onebit_step(st, p16, p32, m32, v32, ew, es, g16)
        bits_w = np.unpackbits(bw, bitorder="little")[:n].astype(np.float64) * 2 - 1
        bits_s = np.unpackbits(bs, bitorder="little")[:n].astype(np.float64) * 2 - 1
        sum_m += m_local
        sum_cw += bits_w * sw
        sum_cs += bits_s * ss
        assert np.array_equal(bits_s * ss, m32.astype(np.float64))  # the momentum is the server output
    tol = 1e-5 * (np.abs(sum_m).max() + 1e-30)
    assert np.abs(sum_cw - (sum_m - ew)).max() <= tol
    assert np.abs(sum_cs - (sum_cw - es)).max() <= tol


def test_skipped_step_changes_nothing(oracle):
    n = 1000
    p16, p32, m32, v32, ew, es = _arrays(8, n)
    m32[:] = 0.5
    ew[:] = 0.25
    g16 = np.zeros(n, np.uint16)
    g16[3] = 0x7C00
    st = _decided(oracle, 8.0, g16)
    snap = [a.copy() for a in (p16, p32, m32, v32, ew, es)]
    bw, bs, sc = oracle.onebit_step(st, p16, p32, m32, v32, ew, es, g16)
    assert st.skip == 1 and sc == (0.0, 0.0)
    for a, b in zip((p16, p32, m32, v32, ew, es), snap):
        assert a.tobytes() == b.tobytes()
