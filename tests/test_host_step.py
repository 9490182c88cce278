"""Parity of the host step (the ZeRO-Offload form: the CPU's exact norm,
decision and AdamW update, AVX-512 on a worker pool) with the oracle, on the
CPU: these run in the CPU suite.

Contract: overflow, skip, loss scale, counters, the exact sum as a 128-bit
integer, sumsq, grad_norm and every fp32 factor bitwise; p16, p32, m32, v32
bitwise (both sides do the same IEEE operations in the same order), for any
thread count, any array alignment and sizes that leave ragged edges."""
import math

import numpy as np
import pytest

import shardgen


@pytest.fixture(scope="module")
def Z():
    import os
    from zero_partitioned_mixed_flatten_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import zero_partitioned_mixed_flatten_amd as Z
    return Z


@pytest.fixture(scope="module")
def ctxs(Z):
    made = {t: Z.HostContext(t) for t in (1, 3, 8)}
    yield made
    for c in made.values():
        c.close()


def _hp(Z, O):
    return Z.hparams(), O.hparams()


def _state_equal(dev, ref, units=None):
    for f in ("loss_scale", "beta1_pow", "beta2_pow", "step", "good_steps", "skipped_total", "overflow", "skip"):
        assert getattr(dev, f) == getattr(ref, f), f
    fields = ("sumsq", "grad_norm") if ref.skip else ("sumsq", "grad_norm", "gmul", "bc1", "bc2", "lr", "beta1",
                                                      "beta2", "omb1", "omb2", "eps", "wd")
    for f in fields:
        assert np.float64(getattr(dev, f)).tobytes() == np.float64(getattr(ref, f)).tobytes(), f
    if units is not None and not ref.skip:
        assert dev.as_dict()["sumsq_units"] == units


def _units(g16):
    """exact sum of squares of finite binary16 values in 2^-48 units (Python ints)."""
    x = g16.view(np.float16).astype(np.float64)
    a = np.abs(x * 2.0 ** 24).astype(np.int64)             # binary16 values are multiples of 2^-24, < 2^40
    lo, hi = a & ((1 << 20) - 1), a >> 20
    return (int((hi * hi).sum()) << 40) + (int((hi * lo).sum()) << 21) + int((lo * lo).sum())


def _offset_view(a, off):
    """a copy of `a` in a buffer starting `off` elements past a 64-byte boundary."""
    buf = np.empty(a.size + off + 64, a.dtype)
    base = (-buf.ctypes.data % 64) // a.itemsize
    v = buf[base + off: base + off + a.size]
    v[:] = a
    return v


@pytest.mark.parametrize("threads", [1, 3, 8])
@pytest.mark.parametrize("n", [0, 1, 31, 32, 33, 4097, 131_072 * 2 + 77, 1_000_003])
def test_norm_matches_oracle(Z, ctxs, threads, n):
    import oracle as O
    rng = np.random.default_rng(n + threads)
    g = shardgen.to_f16_bits((rng.standard_normal(n) * 3000).astype(np.float32))
    st = Z.StepState()
    Z.zero_host_state_init(st, 2.0 ** 16)
    ref = O.new_state(2.0 ** 16)
    hp, hpo = _hp(Z, O)
    Z.zero_host_norm_overflow(ctxs[threads].ptr, g, n, hp, st)
    s, o = O.norm_overflow(g)
    O.decide(ref, hpo, s, o)
    _state_equal(st, ref, _units(g))


def test_norm_extreme_magnitudes_exact(Z, ctxs):
    import oracle as O
    # one 65504 and 2^20 smallest subnormals, across the 4096-iteration flush boundary
    g = np.full((1 << 20) + 1, 0x0001, np.uint16)
    g[0] = 0x7BFF
    st = Z.StepState()
    Z.zero_host_state_init(st, 1.0)
    Z.zero_host_norm_overflow(ctxs[1].ptr, g, g.size, Z.hparams(), st)
    assert st.as_dict()["sumsq_units"] == 65504 ** 2 * 2 ** 48 + (1 << 20)
    assert st.sumsq == O.norm_overflow(g)[0]


@pytest.mark.parametrize("off", [0, 1, 5, 31])
def test_norm_specials_any_alignment(Z, ctxs, off):
    rng = np.random.default_rng(off)
    n = 70_001
    base = shardgen.to_f16_bits((rng.standard_normal(n) * 100).astype(np.float32))
    for pos, val in ((0, 0x7C00), (n - 1, 0xFC00), (33_333, 0x7E01), (None, 0x7BFF)):
        g = base.copy()
        if pos is None:
            g[::9] = val
        else:
            g[pos] = val
        g = _offset_view(g, off)
        st = Z.StepState()
        Z.zero_host_state_init(st, 8.0)
        Z.zero_host_norm_overflow(ctxs[3].ptr, g, n, Z.hparams(), st)
        assert st.overflow == (1 if pos is not None else 0)
        assert st.skip == st.overflow and (math.isinf(st.sumsq) == bool(st.overflow))
        if pos is not None:
            assert st.loss_scale == 4.0 and st.skipped_total == 1


@pytest.mark.parametrize("threads", [1, 8])
@pytest.mark.parametrize("off", [0, 3])
@pytest.mark.parametrize("n", [1, 17, 4096 + 5, 300_007])
def test_adam_matches_oracle_bitwise(Z, ctxs, threads, off, n):
    import oracle as O
    w = shardgen.workload("tiny")
    rng = np.random.default_rng(n * 7 + off)
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp, hpo = _hp(Z, O)
    st = Z.StepState()
    Z.zero_host_state_init(st, w.scale0)
    ref = O.new_state(w.scale0)
    host = [_offset_view(a, off) for a in (shardgen.to_f16_bits(p32), p32, np.zeros_like(p32), np.zeros_like(p32))]
    orc = [shardgen.to_f16_bits(p32), p32.copy(), np.zeros_like(p32), np.zeros_like(p32)]
    for k in range(3):
        g = shardgen.to_f16_bits((rng.standard_normal(n) * 1e-3 * st.loss_scale).astype(np.float32))
        g = _offset_view(g, off)
        Z.zero_host_norm_overflow(ctxs[threads].ptr, g, n, hp, st)
        Z.zero_host_adam_step(ctxs[threads].ptr, *host, g, n, st)
        s, o = O.norm_overflow(np.ascontiguousarray(g))
        O.decide(ref, hpo, s, o)
        O.adam_update(ref, *orc, np.ascontiguousarray(g))
        _state_equal(st, ref)
        for a, b in zip(host, orc):
            assert a.tobytes() == b.tobytes()


def test_adam_skip_writes_nothing(Z, ctxs):
    n = 1000
    rng = np.random.default_rng(2)
    p32 = rng.standard_normal(n).astype(np.float32)
    arrs = [shardgen.to_f16_bits(p32), p32, np.full(n, 0.5, np.float32), np.full(n, 0.25, np.float32)]
    snap = [a.copy() for a in arrs]
    g = shardgen.to_f16_bits(rng.standard_normal(n).astype(np.float32))
    g[10] = 0x7C00
    st = Z.StepState()
    Z.zero_host_state_init(st, 4.0)
    Z.zero_host_norm_overflow(ctxs[8].ptr, g, n, Z.hparams(), st)
    Z.zero_host_adam_step(ctxs[8].ptr, *arrs, g, n, st)
    assert st.skip == 1
    for a, b in zip(arrs, snap):
        assert a.tobytes() == b.tobytes()


def test_fp16_copy_rounding_sweep(Z, ctxs):
    """lr = wd = 0 and a zero gradient leave p32 unchanged, so p16 = fp16(p32)
    through VCVTPS2PH for every exponent and the low-bit patterns around the
    binary16 subnormal/normal/overflow boundaries, against the oracle's own
    converter."""
    import oracle as O
    rng = np.random.default_rng(5)
    parts = [(np.repeat(np.arange(255, dtype=np.uint32), 1 << 10) << 23) |
             rng.integers(0, 1 << 23, 255 << 10, dtype=np.uint32)]
    low = np.arange(1 << 13, dtype=np.uint32)
    for e in range(127 - 27, 127 + 17):
        parts.append((np.uint32(e) << np.uint32(23)) | (np.uint32(rng.integers(0, 1024)) << np.uint32(13)) | low)
    bits = np.concatenate(parts)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    p = bits.view(np.float32).copy()
    n = p.size
    st = Z.StepState()
    Z.zero_host_state_init(st, 1.0)
    hp = Z.hparams(lr=0.0, weight_decay=0.0)
    g = np.zeros(n, np.uint16)
    p16 = np.zeros(n, np.uint16)
    Z.zero_host_norm_overflow(ctxs[8].ptr, g, n, hp, st)
    Z.zero_host_adam_step(ctxs[8].ptr, p16, p, np.zeros(n, np.float32), np.zeros(n, np.float32), g, n, st)
    assert p.view(np.uint32).tobytes() == bits.tobytes()
    assert np.array_equal(p16, O.f16_from_f32(bits.view(np.float32)))


def test_stress_trajectory_through_host_decision(Z, ctxs):
    """The host decision over 100 steps with the stress workload's injections
    (inf at step 3, NaN at step 7) follows the oracle's loss-scale trajectory."""
    import oracle as O
    w = shardgen.workload("stress")
    st = Z.StepState()
    Z.zero_host_state_init(st, w.scale0)
    ref = O.new_state(w.scale0)
    hp, hpo = _hp(Z, O)
    g = np.full(64, 0x3C00, np.uint16)
    for k in range(1, w.steps + 1):
        gk = g.copy()
        if k in w.inject:
            gk[5] = w.inject[k]
        Z.zero_host_norm_overflow(ctxs[3].ptr, gk, gk.size, hp, st)
        O.decide(ref, hpo, *O.norm_overflow(gk))
        _state_equal(st, ref)
    assert (st.loss_scale, st.good_steps, st.step, st.skipped_total) == (2.0 ** 26, 13, 98, 2)


def test_host_stream_copy(Z, ctxs):
    src = np.random.default_rng(1).integers(0, 255, (1 << 22) + 64 * 7, dtype=np.uint8)
    src = _offset_view(src, 0)
    dst = _offset_view(np.zeros_like(src), 0)
    Z.zero_host_stream_copy(ctxs[8].ptr, dst, src, src.size)
    assert dst.tobytes() == src.tobytes()


def test_host_validation(Z, ctxs):
    L, E = Z.lib(), Z._lib
    import ctypes as C
    hp = Z.hparams()
    st = Z.StepState()
    assert L.zero_host_create(1, None) == E.ZERO_EINVAL
    assert L.zero_host_create(5000, C.byref(C.c_void_p())) == E.ZERO_ERANGE
    assert L.zero_host_state_init(C.byref(st), 0.0) == E.ZERO_EINVAL
    assert L.zero_host_norm_overflow(None, 0, 0, C.byref(hp), C.byref(st)) == E.ZERO_EINVAL
    assert L.zero_host_norm_overflow(ctxs[1].ptr, None, 5, C.byref(hp), C.byref(st)) == E.ZERO_EINVAL
    bad = Z.hparams(eps=0.0)
    assert L.zero_host_norm_overflow(ctxs[1].ptr, None, 0, C.byref(bad), C.byref(st)) == E.ZERO_EINVAL
    assert L.zero_host_adam_step(ctxs[1].ptr, None, None, None, None, None, 3, C.byref(st)) == E.ZERO_EINVAL
    assert L.zero_host_stream_copy(ctxs[1].ptr, 64, 128, 63) == E.ZERO_EALIGN
    assert L.zero_host_stream_copy(ctxs[1].ptr, 65, 128, 64) == E.ZERO_EALIGN
    # the offload step rejects a bad chunk before touching the device
    f = 1 << 20
    sp = C.addressof(st)
    assert L.zero_offload_step(ctxs[1].ptr, f, f, f, f, f, f, f, 100, C.byref(hp), sp, None, 100,
                               None) == E.ZERO_EALIGN
    assert L.zero_offload_step(ctxs[1].ptr, f, f, f, f, f, f, f, 1 << 30, C.byref(hp), sp, None, 64,
                               None) == E.ZERO_ERANGE
    assert L.zero_offload_step(ctxs[1].ptr, f, f, f, f, f, f, f, 100, None, sp, None, 64,
                               None) == E.ZERO_EINVAL             # no hp and no device decision
    assert L.zero_offload_step(ctxs[1].ptr, f, f, f, f, f, f, f, 100, None, sp, f + 4, 64,
                               None) == E.ZERO_EALIGN             # misaligned device state
    assert Z.zero_status_string(E.ZERO_ENOTSUP) and Z.zero_status_string(E.ZERO_ENOMEM)


# ---- randomized: any size, alignment, worker count, gradient pattern and hyperparameters ----

from hypothesis import HealthCheck, given, settings, strategies as hs  # noqa: E402


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(n=hs.integers(0, 3000), off=hs.integers(0, 31), threads=hs.sampled_from([1, 3, 8]),
       seed=hs.integers(0, 2 ** 32 - 1), special=hs.sampled_from([None, 0x7C00, 0xFE00, 0x7BFF, 0x0001]),
       lr=hs.floats(0.0, 1e-2), b1=hs.floats(0.0, 0.999), b2=hs.floats(0.0, 0.9999),
       wd=hs.floats(0.0, 0.1), clip=hs.sampled_from([0.0, 1e-3, 1.0]), scale_exp=hs.integers(0, 24))
def test_host_step_random_against_oracle(Z, ctxs, n, off, threads, seed, special, lr, b1, b2, wd, clip, scale_exp):
    import oracle as O
    rng = np.random.default_rng(seed)
    S = 2.0 ** scale_exp
    g = shardgen.to_f16_bits((rng.standard_normal(n) * rng.choice([1e-3, 1.0, 100.0])).astype(np.float32))
    if special is not None and n:
        g[int(rng.integers(n))] = special
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m32 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v32 = (np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32)
    host = [_offset_view(a, off) for a in (shardgen.to_f16_bits(p32), p32, m32, v32)]
    orc = [shardgen.to_f16_bits(p32), p32.copy(), m32.copy(), v32.copy()]
    gv = _offset_view(g, off)
    hp = Z.hparams(lr=lr, beta1=b1, beta2=b2, weight_decay=wd, max_grad_norm=clip)
    hpo = O.hparams(lr=lr, beta1=b1, beta2=b2, weight_decay=wd, max_grad_norm=clip)
    st = Z.StepState()
    Z.zero_host_state_init(st, S)
    ref = O.new_state(S)
    Z.zero_host_norm_overflow(ctxs[threads].ptr, gv, n, hp, st)
    Z.zero_host_adam_step(ctxs[threads].ptr, *host, gv, n, st)
    s, o = O.norm_overflow(g)
    O.decide(ref, hpo, s, o)
    O.adam_update(ref, *orc, g)
    _state_equal(st, ref)
    for a, b in zip(host, orc):
        assert a.tobytes() == b.tobytes()


def test_host_f32_is_zeroed_aligned_and_writable():
    import torch

    from zero_partitioned_mixed_flatten_amd.stepper import host_f32
    for huge in (True, False):
        t = host_f32(3_000_007, huge)
        assert t.dtype == torch.float32 and t.numel() == 3_000_007 and not t.any()
        if huge:
            assert t.data_ptr() % (2 << 20) == 0
        v = t[5:17]                                   # a view keeps the mapping alive with its storage
        del t
        v.fill_(2.5)
        assert float(v.sum()) == 30.0
