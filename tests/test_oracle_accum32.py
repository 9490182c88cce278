"""Pins for the oracle's fp32-gradient (gradient-accumulation) reduction and
update.

The reduction's definition: overflow iff some element is inf or NaN; otherwise
the sum of the squares, every square and the sum exact, rounded once to
binary64.  It is checked against
  * exact rational sums (fractions.Fraction, whose float() rounds correctly),
    on vectors of the accumulation domain and on binary32 vectors drawn over
    the whole binary32 range, subnormals and the largest finite values
    included;
  * math.fsum (a correctly rounded sum; every binary32 square is exact in
    binary64) on large vectors;
  * the binary16 reduction (itself pinned) on the widened binary16 values;
  * every class of special value.
The update is checked against closed forms of Adam with decoupled weight decay
and against the binary16 update on the widened gradient."""
import math
from fractions import Fraction

import numpy as np
import pytest

import shardgen

LR, B1, B2, EPS, WD = 1e-4, 0.9, 0.999, 1e-8, 0.01
S16 = 2.0 ** 16
F32_MAX = float(np.finfo(np.float32).max)


def _accumulated(rng, n, k, spread=300.0):
    """binary32 sums of k binary16 values, accumulated in binary32 like the flatten."""
    acc = np.zeros(n, np.float32)
    for _ in range(k):
        h = (rng.standard_normal(n) * spread).astype(np.float16)
        acc = acc + h.astype(np.float32)
    return acc


def _exact(x32):
    """The exact sum of squares as a rational, rounded once by float()."""
    return float(sum((Fraction(float(v)) ** 2 for v in x32.astype(np.float64)), Fraction(0)))


def _any_f32(rng, n, lo=-149, hi=127):
    """Finite binary32 values with random significands, exponents in [lo, hi]
    (values below 2^-126 come out subnormal), random signs."""
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    expo = rng.integers(lo, hi + 1, n).astype(np.float64)
    x = mant * np.exp2(expo - 23)
    x = np.where(x > F32_MAX, F32_MAX, x).astype(np.float32)
    return x * np.where(rng.integers(0, 2, n) == 1, -1, 1).astype(np.float32)


@pytest.mark.parametrize("seed", range(5))
def test_domain_sum_is_exact(oracle, seed):
    rng = np.random.default_rng(seed)
    x = _accumulated(rng, int(rng.integers(1, 400)), int(rng.integers(1, 9)))
    s, ovf = oracle.norm_overflow_f32(x)
    assert ovf == 0 and s == _exact(x)


@pytest.mark.parametrize("seed,lo,hi", [(0, -149, 127), (1, -149, 127), (2, -149, -100), (3, -60, 30),
                                        (4, 100, 127), (5, -149, 127)])
def test_any_binary32_sum_is_exact(oracle, seed, lo, hi):
    # squares from 2^-298 (the smallest subnormal, squared) up to about 2^256
    rng = np.random.default_rng(50 + seed)
    x = _any_f32(rng, 300, lo, hi)
    s, ovf = oracle.norm_overflow_f32(x)
    assert ovf == 0 and s == _exact(x)


def test_tiny_squares_far_below_the_largest_still_count(oracle):
    # 1 + 2 * 2^-54 is exactly halfway between 1 and 1 + 2^-52; the 2^-120
    # from the last element breaks the tie upward.  A sum that dropped squares
    # that far below the largest would round to 1.
    x = np.array([1.0, 2.0 ** -27, -(2.0 ** -27), 2.0 ** -60], np.float32)
    assert oracle.norm_overflow_f32(x) == (1.0 + 2.0 ** -52, 0)
    assert oracle.norm_overflow_f32(x[:3]) == (1.0, 0)              # the exact tie goes to even
    y = np.array([2.0 ** -149, -(2.0 ** -149), 2.0 ** -140], np.float32)
    assert oracle.norm_overflow_f32(y)[0] == 2 * 2.0 ** -298 + 2.0 ** -280


@pytest.mark.parametrize("seed", range(2))
def test_fsum_large(oracle, seed):
    rng = np.random.default_rng(70 + seed)
    for x in (_accumulated(rng, 100_000, 4, spread=3000.0), _any_f32(rng, 100_000)):
        xd = x.astype(np.float64)
        s, ovf = oracle.norm_overflow_f32(x)
        assert ovf == 0 and s == math.fsum(xd * xd)                 # squares exact in binary64


@pytest.mark.parametrize("seed", range(3))
def test_agrees_with_binary16_reduction_on_widened_values(oracle, seed):
    rng = np.random.default_rng(90 + seed)
    h = rng.integers(0, 1 << 16, 20_000).astype(np.uint16)
    h = h[(h & 0x7C00) != 0x7C00]
    assert oracle.norm_overflow_f32(oracle.f32_from_f16(h)) == oracle.norm_overflow(h)
    h[123] = 0xFC00                                 # -inf
    assert oracle.norm_overflow_f32(oracle.f32_from_f16(h)) == (math.inf, 1)


def test_large_finite_values_are_summed_inf_flags(oracle):
    top = np.float32(2.0 ** 24)
    x = np.array([1.0, top, -np.float32(F32_MAX), 2.0], np.float32)
    s, ovf = oracle.norm_overflow_f32(x)
    assert ovf == 0 and s == _exact(x) and s > 1e76
    for bad in (np.float32(np.inf), np.float32(-np.inf)):
        y = np.array([1.0, bad, 2.0], np.float32)
        assert oracle.norm_overflow_f32(y) == (math.inf, 1)


def test_every_nan_class_flags(oracle):
    bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0x7FA00000], np.uint32)
    for b in bits:
        x = np.array([0.5, 0.25, 0.0], np.float32)
        x.view(np.uint32)[1] = b
        assert oracle.norm_overflow_f32(x) == (math.inf, 1)


def test_empty_and_signed_zeros(oracle):
    assert oracle.norm_overflow_f32(np.zeros(0, np.float32)) == (0.0, 0)
    assert oracle.norm_overflow_f32(np.array([0.0, -0.0], np.float32)) == (0.0, 0)


# ---- the update reading an fp32 gradient --------------------------------------------

def _state(seed, n, sigma=0.02):
    rng = np.random.default_rng(seed)
    p32 = (rng.standard_normal(n) * sigma).astype(np.float32)
    return p32, np.zeros(n, np.float32), np.zeros(n, np.float32), shardgen.to_f16_bits(p32)


def _close(got, ref, scale, tol=1e-6):
    err = np.abs(got.astype(np.float64) - ref)
    bound = tol * np.maximum(scale, np.abs(ref)) + 1e-30
    assert np.all(err <= bound), float(np.max(err / bound))


def _step32(oracle, st, hp, g32, p16, p32, m32, v32):
    s, o = oracle.norm_overflow_f32(g32)
    oracle.decide(st, hp, s, o)
    oracle.adam_update_f32(st, p16, p32, m32, v32, g32)


def test_widened_binary16_gradient_gives_the_binary16_update_bitwise(oracle):
    w = shardgen.workload("tiny")
    p32a = shardgen.master_params(w)
    m_a, v_a = np.zeros_like(p32a), np.zeros_like(p32a)
    p16a = shardgen.to_f16_bits(p32a)
    p32b, m_b, v_b, p16b = p32a.copy(), m_a.copy(), v_a.copy(), p16a.copy()
    hp = oracle.hparams()
    sa, sb = oracle.new_state(w.scale0), oracle.new_state(w.scale0)
    for k in range(1, 4):
        g16 = shardgen.grad_partition(w, k, sa.loss_scale)
        s, o = oracle.norm_overflow(g16)
        oracle.decide(sa, hp, s, o)
        oracle.adam_update(sa, p16a, p32a, m_a, v_a, g16)
        _step32(oracle, sb, hp, oracle.f32_from_f16(g16), p16b, p32b, m_b, v_b)
        assert sa.as_dict() == sb.as_dict()
    for a, b in ((p16a, p16b), (p32a, p32b), (m_a, m_b), (v_a, v_b)):
        assert a.tobytes() == b.tobytes()


def test_first_step_closed_form_fp32_gradient(oracle):
    n = 4096
    rng = np.random.default_rng(3)
    g32 = (rng.standard_normal(n) * 1e-3 * S16).astype(np.float32)   # not binary16 values
    g = g32.astype(np.float64) / S16
    p32, m32, v32, p16 = _state(4, n)
    p0 = p32.astype(np.float64)
    st = oracle.new_state(S16)
    _step32(oracle, st, oracle.hparams(lr=LR, max_grad_norm=0.0), g32, p16, p32, m32, v32)
    _close(p32, p0 - LR * (g / (np.abs(g) + EPS) + WD * p0), np.abs(p0))
    _close(m32, (1 - B1) * g, 0)
    _close(v32, (1 - B2) * g * g, 0)
    assert np.array_equal(p16, shardgen.to_f16_bits(p32))


def test_accumulated_microbatches_step_on_their_sum(oracle):
    # Micro-batch gradients of small integers times 2^-10 add exactly in fp32,
    # so the accumulated step must be Adam on the exact sum (closed form).
    n, k = 2048, 6
    rng = np.random.default_rng(5)
    parts = [(rng.integers(-40, 41, n) * 2.0 ** -10).astype(np.float16).view(np.uint16) for _ in range(k)]
    acc = np.zeros(n, np.float32)
    oracle.flatten([parts[0]], [(0, 0, 0, n)], acc, accumulate=False)
    for h in parts[1:]:
        oracle.flatten([h], [(0, 0, 0, n)], acc, accumulate=True)
    total = sum(h.view(np.float16).astype(np.float64) for h in parts)
    assert np.array_equal(acc.astype(np.float64), total)
    p32, m32, v32, p16 = _state(6, n)
    p0 = p32.astype(np.float64)
    st = oracle.new_state(1.0)
    _step32(oracle, st, oracle.hparams(lr=LR, max_grad_norm=0.0), acc, p16, p32, m32, v32)
    assert st.sumsq == float(sum(Fraction(float(t)) ** 2 for t in total))
    g = total
    upd = np.where(g != 0, g / (np.abs(g) + EPS), 0.0)
    _close(p32, p0 - LR * (upd + WD * p0), np.abs(p0))


def test_clip_brings_fp32_norm_to_threshold(oracle):
    n = 1 << 15
    rng = np.random.default_rng(7)
    g32 = (rng.standard_normal(n) * 0.05 * S16).astype(np.float32)
    st = oracle.new_state(S16)
    s, o = oracle.norm_overflow_f32(g32)
    oracle.decide(st, oracle.hparams(max_grad_norm=1.0), s, o)
    gd = g32.astype(np.float64)
    true_norm = math.sqrt(math.fsum(gd * gd)) / S16
    assert true_norm > 1.0 and st.grad_norm == pytest.approx(true_norm, rel=1e-12)
    applied = gd * float(np.float32(st.gmul))
    assert math.sqrt(math.fsum(applied * applied)) == pytest.approx(1.0, rel=1e-6)


def test_huge_finite_fp32_gradient_is_clipped_not_skipped(oracle):
    # A finite gradient far beyond anything binary16 can hold is a gradient
    # like any other: the step applies, clipped to the threshold.
    n = 1000
    rng = np.random.default_rng(8)
    g32 = rng.standard_normal(n).astype(np.float32)
    g32[500] = np.float32(3e38)
    p32, m32, v32, p16 = _state(9, n)
    st = oracle.new_state(S16)
    _step32(oracle, st, oracle.hparams(), g32, p16, p32, m32, v32)
    gd = g32.astype(np.float64)
    assert st.skip == 0 and st.overflow == 0 and st.step == 1 and st.loss_scale == S16
    assert st.sumsq == math.fsum(gd * gd) and st.grad_norm == math.sqrt(st.sumsq) / S16
    assert st.gmul == np.float32(1.0 / st.grad_norm / S16)


def test_nan_tolerant_comparison_of_accumulated_gradients():
    """The GPU harness compares accumulated binary32 gradients bit for bit but
    lets an element that is NaN on both sides carry any NaN bits (IEEE 754
    leaves a NaN result's sign and payload unspecified); a NaN on one side
    only, or any other bit difference, still fails."""
    from floatcmp import same_floats32 as same
    a = np.array([1.0, -0.0, np.inf, np.nan], np.float32)
    b = a.copy()
    b.view(np.uint32)[3] = 0xFFC00000                       # another NaN: matches
    assert same(a, b)
    c = a.copy(); c[1] = 0.0                                 # -0.0 vs +0.0: differs
    assert not same(a, c)
    d = a.copy(); d[0] = np.nan                              # NaN on one side only
    assert not same(a, d)
    e = a.copy(); e.view(np.uint32)[0] += 1                  # one ulp
    assert not same(a, e)
