"""Pins for the oracle's step decision and AdamW element update.

Nothing here re-types the oracle's recurrence.  The checks are:
  * closed forms of Adam (Kingma & Ba 2015) with decoupled weight decay
    (Loshchilov & Hutter 2019) that follow from the definition: first step
    from zero moments, t steps of a constant gradient, two distinct steps;
  * bitwise special cases (zero gradient, zero weight decay);
  * the clipped gradient's norm equals the threshold (Pascanu et al. 2013);
  * the loss-scale trajectory of the stress workload in closed form
    (Micikevicius et al. 2018: skip and halve on overflow, double after 20
    clean steps);
  * the fp16 parameter copy against numpy's float16 cast.
Tolerance for fp32 state against fp64 closed forms: 1e-6 relative to the
operands' scale."""
import math

import numpy as np
import pytest

import shardgen

LR, B1, B2, EPS, WD = 1e-4, 0.9, 0.999, 1e-8, 0.01
S16 = 2.0 ** 16


def _grads(seed, n, sigma=1e-3, scale=S16):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(n).astype(np.float32) * np.float32(sigma)
    g16 = shardgen.to_f16_bits(g * np.float32(scale))
    g_real = g16.view(np.float16).astype(np.float64) / scale      # exact unscaled value
    return g16, g_real


def _state(seed, n, sigma=0.02):
    rng = np.random.default_rng(seed)
    p32 = (rng.standard_normal(n) * sigma).astype(np.float32)
    return p32, np.zeros(n, np.float32), np.zeros(n, np.float32), shardgen.to_f16_bits(p32)


def _step(oracle, st, hp, g16, p16, p32, m32, v32):
    s, o = oracle.norm_overflow(g16)
    oracle.decide(st, hp, s, o)
    oracle.adam_update(st, p16, p32, m32, v32, g16)


def _close(got, ref, scale, tol=1e-6):
    err = np.abs(got.astype(np.float64) - ref)
    bound = tol * np.maximum(scale, np.abs(ref)) + 1e-30
    assert np.all(err <= bound), float(np.max(err / bound))


def test_first_step_closed_form(oracle):
    n = 4096
    g16, g = _grads(1, n)
    p32, m32, v32, p16 = _state(2, n)
    p0 = p32.astype(np.float64)
    hp = oracle.hparams(lr=LR, max_grad_norm=0.0)
    st = oracle.new_state(S16)
    _step(oracle, st, hp, g16, p16, p32, m32, v32)
    # from zero moments the bias corrections cancel: m_hat = g, v_hat = g^2
    p1 = p0 - LR * (g / (np.abs(g) + EPS) + WD * p0)
    _close(p32, p1, np.abs(p0))
    _close(m32, (1 - B1) * g, 0)
    _close(v32, (1 - B2) * g * g, 0)
    assert st.step == 1 and st.skip == 0


def test_constant_gradient_t_steps(oracle):
    n, T = 4096, 20
    g16, g = _grads(3, n)
    p32, m32, v32, p16 = _state(4, n)
    p0 = p32.astype(np.float64)
    hp = oracle.hparams(lr=LR, max_grad_norm=0.0, growth_interval=0)
    st = oracle.new_state(S16)
    for _ in range(T):
        _step(oracle, st, hp, g16, p16, p32, m32, v32)
    # m_t = (1-b1^t) g and v_t = (1-b2^t) g^2, so m_hat = g and sqrt(v_hat) = |g|
    # every step, and p follows p_t = a p_{t-1} - lr s with a = 1 - lr*wd:
    a = 1.0 - LR * WD
    s = g / (np.abs(g) + EPS)
    pT = a ** T * p0 - LR * s * (1 - a ** T) / (1 - a)
    _close(p32, pT, np.abs(p0))
    _close(m32, (1 - B1 ** T) * g, 0)
    _close(v32, (1 - B2 ** T) * g * g, 0)
    assert st.step == T
    assert abs(st.beta1_pow - B1 ** T) <= 1e-15 and abs(st.beta2_pow - B2 ** T) <= 1e-15


def test_two_distinct_steps(oracle):
    n = 4096
    g16a, g1 = _grads(5, n)
    g16b, g2 = _grads(6, n)
    p32, m32, v32, p16 = _state(7, n)
    p0 = p32.astype(np.float64)
    hp = oracle.hparams(lr=LR, max_grad_norm=0.0)
    st = oracle.new_state(S16)
    _step(oracle, st, hp, g16a, p16, p32, m32, v32)
    _step(oracle, st, hp, g16b, p16, p32, m32, v32)
    mhat2 = (B1 * g1 + g2) / (1 + B1)                 # (1-b1)(b1 g1 + g2) / (1-b1^2)
    vhat2 = (B2 * g1 * g1 + g2 * g2) / (1 + B2)
    p1 = p0 - LR * (g1 / (np.abs(g1) + EPS) + WD * p0)
    p2 = p1 - LR * (mhat2 / (np.sqrt(vhat2) + EPS) + WD * p1)
    _close(p32, p2, np.abs(p0))
    _close(m32, (1 - B1) * (B1 * g1 + g2), (1 - B1) * (B1 * np.abs(g1) + np.abs(g2)))
    _close(v32, (1 - B2) * (B2 * g1 * g1 + g2 * g2), 0)


def test_zero_gradient_zero_decay_leaves_params_bitwise(oracle):
    n = 1000
    p32, m32, v32, p16 = _state(8, n)
    before = p32.copy()
    st = oracle.new_state(S16)
    _step(oracle, st, oracle.hparams(weight_decay=0.0), np.zeros(n, np.uint16), p16, p32, m32, v32)
    assert np.array_equal(p32.view(np.uint32), before.view(np.uint32))
    assert np.array_equal(p16, shardgen.to_f16_bits(before))
    assert not m32.any() and not v32.any()


def test_zero_gradient_pure_decay(oracle):
    n = 1000
    p32, m32, v32, p16 = _state(9, n)
    p0 = p32.astype(np.float64)
    st = oracle.new_state(S16)
    _step(oracle, st, oracle.hparams(), np.zeros(n, np.uint16), p16, p32, m32, v32)
    assert not m32.any() and not v32.any()
    _close(p32, p0 * (1 - LR * WD), np.abs(p0))


def test_descends_along_the_gradient(oracle):
    n = 2000
    g16, g = _grads(10, n)
    p32, m32, v32, p16 = _state(11, n)
    p0 = p32.copy()
    st = oracle.new_state(S16)
    _step(oracle, st, oracle.hparams(weight_decay=0.0, max_grad_norm=0.0), g16, p16, p32, m32, v32)
    moved = g != 0
    assert np.all(np.sign(p0[moved] - p32[moved]) == np.sign(g[moved]))


def test_clip_brings_norm_to_threshold(oracle):
    n = 1 << 16
    g16, g = _grads(12, n, sigma=1e-2)                 # norm ~ 2.56 > 1
    st = oracle.new_state(S16)
    s, o = oracle.norm_overflow(g16)
    oracle.decide(st, oracle.hparams(max_grad_norm=1.0), s, o)
    true_norm = math.sqrt(math.fsum(g * g))
    assert st.grad_norm == pytest.approx(true_norm, rel=1e-12) and true_norm > 1.0
    applied = g16.view(np.float16).astype(np.float64) * float(np.float32(st.gmul))
    assert math.sqrt(math.fsum(applied * applied)) == pytest.approx(1.0, rel=1e-6)


def test_no_clip_below_threshold_is_exact_unscale(oracle):
    n = 1 << 12
    g16, g = _grads(13, n)                             # norm ~ 0.064 < 1
    for clip in (1.0, 0.0):
        st = oracle.new_state(S16)
        s, o = oracle.norm_overflow(g16)
        oracle.decide(st, oracle.hparams(max_grad_norm=clip), s, o)
        assert np.float32(st.gmul) == np.float32(1.0 / S16)


def test_clip_tie_does_not_clip(oracle):
    # a gradient whose unscaled norm is exactly 1.0: 1 element of value S
    st = oracle.new_state(S16)
    g16 = shardgen.to_f16_bits(np.array([1.0], np.float32))
    s, o = oracle.norm_overflow(g16)
    oracle.decide(st, oracle.hparams(max_grad_norm=1.0 * 2 ** -16), s, o)   # norm == clip
    assert np.float32(st.gmul) == np.float32(1.0 / S16)


def test_stress_loss_scale_trajectory_closed_form(oracle):
    w = shardgen.workload("stress")
    st = oracle.new_state(w.scale0)
    hp = oracle.hparams()
    traj = []
    for k in range(1, w.steps + 1):
        oracle.decide(st, hp, 1.0, 1 if k in w.inject else 0)
        traj.append((st.loss_scale, st.skip))
    S = lambda e: 2.0 ** e
    assert traj[0] == (S(24), 0) and traj[1] == (S(24), 0)
    assert traj[2] == (S(23), 1)                       # inf at step 3: skip, halve
    assert traj[3:6] == [(S(23), 0)] * 3
    assert traj[6] == (S(22), 1)                       # NaN at step 7: skip, halve
    # 20 clean steps after step 7 -> growth after steps 27, 47, 67, 87
    for k, e in ((26, 22), (27, 23), (46, 23), (47, 24), (66, 24), (67, 25), (86, 25), (87, 26), (100, 26)):
        assert traj[k - 1][0] == S(e), k
    assert st.loss_scale == S(26) and st.good_steps == 13 and st.step == 98 and st.skipped_total == 2


def test_scale_floor_and_no_growth(oracle):
    st = oracle.new_state(1.0)
    oracle.decide(st, oracle.hparams(), 1.0, 1)
    assert st.loss_scale == 1.0 and st.skip == 1 and st.step == 0
    st = oracle.new_state(4.0)
    for _ in range(100):
        oracle.decide(st, oracle.hparams(growth_interval=0), 1.0, 0)
    assert st.loss_scale == 4.0 and st.step == 100


def test_skipped_step_changes_nothing(oracle):
    n = 3000
    g16, _ = _grads(14, n)
    g16[1234] = 0x7C00
    p32, m32, v32, p16 = _state(15, n)
    m32[:] = 0.5
    v32[:] = 0.25
    snap = [a.copy() for a in (p16, p32, m32, v32)]
    st = oracle.new_state(S16)
    _step(oracle, st, oracle.hparams(), g16, p16, p32, m32, v32)
    assert st.skip == 1 and st.overflow == 1 and st.step == 0 and st.loss_scale == S16 / 2
    for a, b in zip((p16, p32, m32, v32), snap):
        assert a.tobytes() == b.tobytes()


def test_fp16_copy_is_numpy_cast_over_steps(oracle):
    w = shardgen.workload("tiny")
    p32 = shardgen.master_params(w)
    m32, v32 = np.zeros_like(p32), np.zeros_like(p32)
    p16 = shardgen.to_f16_bits(p32)
    st = oracle.new_state(w.scale0)
    hp = oracle.hparams()
    srcs = None
    for k in range(1, 4):
        gpart = shardgen.grad_partition(w, k, st.loss_scale)
        srcs = shardgen.source_tensors(w.layout, gpart)
        grad16 = np.empty(w.n, np.uint16)
        oracle.step(hp, st, srcs, w.layout.segments, grad16, p16, p32, m32, v32)
        assert np.array_equal(grad16, gpart)
        assert np.array_equal(p16, shardgen.to_f16_bits(p32))
        assert st.skip == 0 and st.grad_norm > 1.0       # the tiny workload always clips
    assert st.step == 3
