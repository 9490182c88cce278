"""GPU parity tests of the gradient-accumulation form: K micro-batches of
per-layer fp16 gradients added into an fp32 partition, the fp32 exact
reduction (standalone, or fused into the last micro-batch's flatten), the
decision and the update reading the fp32 gradient -- through the C ABI,
against the CPU oracle on the same seeded inputs.  Contract as in
tests/gpu_harness.py: accumulated gradient bitwise, step state bitwise
(including the exact sum as a 128-bit integer), p16 bitwise, fp32 state
within 1e-6 relative (0 elements differing expected)."""
import numpy as np
import pytest
import torch

import oracle as O
import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _small(name, n, seed, max_seg=None, misalign=True):
    w = shardgen.workload("tiny")
    w.name = name
    rng = np.random.default_rng(seed)
    numels, segs = shardgen.random_segments(rng, n, max_seg or max(1, n // 5), misalign)
    w.layout = shardgen.ShardLayout(name, n, 1, 0, 0, n, [f"t{i}" for i in range(len(numels))], numels, segs)
    return w


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("micro", [1, 3])
def test_accum_tiny_workload_full_parity(fused, micro):
    w = shardgen.workload("tiny")
    r = H.start_accum(w, micro, fused=fused)
    for _ in range(4):
        H.step_accum(r)
    assert r.st.step == 4 and r.stats["fp32_not_bitwise"] == 0, r.stats
    H.log(f"accum tiny micro={micro} fused={fused}: {r.stats}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("n", [1, 7, 9, 4099, 65_536 * 3 + 5, (1 << 20) + 3])
def test_accum_ragged_sizes_misaligned_segments(n, fused):
    w = _small(f"accum-ragged{n}", n, seed=100 + n)
    r = H.start_accum(w, 2, fused=fused)
    for _ in range(2):
        H.step_accum(r)
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


def test_accum_empty_shard():
    w = _small("accum-empty", 0, seed=0)
    w.layout = shardgen.ShardLayout("empty", 0, 1, 0, 0, 0, [], [], [])
    for fused in (False, True):
        r = H.start_accum(w, 2, fused=fused)
        H.step_accum(r)
        s = r.dev.read_state()
        assert s.sumsq == 0.0 and s.step == 1 and s.overflow == 0


@pytest.mark.parametrize("fused", [False, True])
def test_accum_gpt2_shard_full_size(fused):
    w = shardgen.workload("gpt2")
    r = H.start_accum(w, 4, sample=1 << 20, fused=fused)
    for _ in range(2):
        H.step_accum(r)
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.timeout(900)
def test_accum_1t_shard_bucketed():
    w = shardgen.workload("1t")
    r = H.start_accum(w, 2, sample=1 << 18, fused=True)
    H.step_accum(r)


def test_accum_fused_and_separate_identical():
    w = _small("accum-fused-vs-separate", 2_000_003, seed=41, max_seg=300_000)
    w.bucket_elems = 700_000
    runs = [H.start_accum(w, 3, fused=f) for f in (False, True)]
    for _ in range(2):
        for r in runs:
            H.step_accum(r)
        a, b = (r.dev.read_state() for r in runs)
        assert bytes(a) == bytes(b)
    for x, y in zip((runs[0].dev.grad32, runs[0].dev.p32, runs[0].dev.m32),
                    (runs[1].dev.grad32, runs[1].dev.p32, runs[1].dev.m32)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def _crafted_f32(n, seed, lo=-80, hi=1, top=16777215.0):
    """binary32 values with random significands and exponents in [lo, hi)
    (most off the 2^-24 grid), random signs, plus `top` every 97th element."""
    rng = np.random.default_rng(seed)
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    expo = rng.integers(lo, hi, n).astype(np.float64)
    x = np.minimum(mant * np.exp2(expo), float(np.finfo(np.float32).max)).astype(np.float32)
    x *= np.where(rng.integers(0, 2, n) == 1, -1, 1).astype(np.float32)
    x[::97] = np.float32(top)
    x[1::101] = np.float32(3 * 2.0 ** -26)
    return x


def _units48(g32):
    """The exact sum of squares in 2^-48 units when it is a whole number of
    them below 2^128, else the all-ones sentinel: Python integers, from the
    IEEE binary32 fields (x = M * 2^e)."""
    b = g32.view(np.uint32) & np.uint32(0x7FFFFFFF)
    field = (b >> np.uint32(23)).astype(np.int64)
    mant = (b & np.uint32(0x7FFFFF)).astype(np.int64) | np.where(field > 0, 1 << 23, 0)
    e = np.where(field > 0, field - 150, -149)
    total = 0                                        # in units of 2^-298
    for m, k in zip(mant.tolist(), (2 * e + 298).tolist()):
        total += (m * m) << k
    if total % (1 << 250):
        return (1 << 128) - 1
    u = total >> 250
    return u if u < (1 << 128) else (1 << 128) - 1


def _decide_standalone(g32):
    n = g32.size
    ws = torch.empty(max(16, Z.zero_norm_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st, 1024.0)
    Z.zero_shard_norm_overflow_f32(torch.from_numpy(g32).cuda(), n, Z.hparams(), st, ws)
    return Z.read_state(st)


def _check_sum(s, g, scale0=1024.0):
    sumsq, ovf = O.norm_overflow_f32(g)
    assert s.overflow == ovf and s.wide_pending == 0
    assert np.float64(s.sumsq).tobytes() == np.float64(sumsq).tobytes(), (s.sumsq, sumsq)
    if not ovf:
        ref = O.new_state(scale0)
        O.decide(ref, O.hparams(), sumsq, ovf)
        H.compare_state(s, ref, _units48(g) if g.size <= 300_000 else None)
    return ovf


@pytest.mark.parametrize("n,lo,hi", [(5, -149, 128), (4096 * 3 + 1, -149, 128), (4096 * 3 + 1, -149, -120),
                                     (1_000_003, -80, 1), (1_000_003, -40, -32), (65_537, 100, 128)])
def test_norm_f32_exact_over_the_whole_binary32_range(n, lo, hi):
    """Values off the fast path (off the 2^-24 grid, subnormal, up to the
    largest binary32) go through the wide pass: the decision and the exact
    sum bit for bit against the oracle."""
    g = _crafted_f32(n, seed=n + lo + 1000, lo=lo, hi=hi, top=2.0 ** (hi - 1) if hi < 24 else 16777215.0)
    H.log(f"norm f32 crafted n={n} exponents [{lo}, {hi})")
    _check_sum(_decide_standalone(g), g)


def test_norm_f32_tie_needs_every_square():
    # 1 + 2 * 2^-54 is halfway between two binary64 values; the square of
    # 2^-60 (2^-120) breaks the tie upward -- only an exact sum sees it
    for n in (4, 50_000, 1_000_000):
        g = np.zeros(n, np.float32)
        g[[0, n // 3, n // 2, n - 1]] = [1.0, 2.0 ** -27, -(2.0 ** -27), 2.0 ** -60]
        s = _decide_standalone(g)
        assert s.sumsq == 1.0 + 2.0 ** -52
        _check_sum(s, g)


def test_norm_f32_special_values_everywhere():
    n = 4 * 5000 + 3
    rng = np.random.default_rng(6)
    # sums of two binary16 values: on the 2^-24 grid, so the exact sum is checkable
    base = sum((rng.standard_normal(n) * 1000).astype(np.float16).astype(np.float32) for _ in range(2))
    cases = [(0, np.inf), (n - 1, -np.inf), (n - 2, np.nan), (777, 2.0 ** 24), (4 * 4999, -(2.0 ** 24)),
             (31, 3e38), (None, 16777215.0)]
    for pos, val in cases:
        g = base.copy()
        if pos is None:
            g[::5] = val
        else:
            g[pos] = val
        H.log(f"norm f32 special pos={pos} val={val}")
        ovf = _check_sum(_decide_standalone(g), g)
        assert ovf == (1 if not np.isfinite(val) else 0)


def test_fused_f32_accumulate_into_crafted_partition():
    """The fused fp32 flatten sums squares of the values it stores, and
    zero_shard_decide_f32 completes the sum with the wide pass when a value is
    off the fast path: a partition holding off-grid values, and one where the
    added micro-batch lands a value exactly on 2^24.  Folded by
    zero_shard_decide alone, such partials leave the step pending: skipped,
    loss scale and counters untouched."""
    rng = np.random.default_rng(44)
    n = 300_007
    numels, segs = shardgen.random_segments(rng, n, 40_000)
    srcs = [shardgen.to_f16_bits((rng.standard_normal(k) * 20).astype(np.float32)) for k in numels]
    dsrcs = [H.to_dev16(s) for s in srcs]
    arr, k = Z.make_segments([(dsrcs[t].data_ptr(), so, do, c) for t, so, do, c in segs])
    count = Z.zero_flatten_norm_partials(arr, k)
    partials = torch.empty(count * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(16, Z.zero_decide_workspace_bytes(count)), dtype=torch.uint8, device="cuda")
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    flat = np.concatenate([srcs[t][so:so + c] for t, so, _, c in segs]).view(np.float16).astype(np.float32)
    base = _crafted_f32(n, seed=45, top=2.0 ** 23)             # room for the added micro-batch
    pos = int(np.argmax(flat > 0))
    cases = [("off-grid", base)]
    over = base.copy()
    over[pos] = np.float32(2.0 ** 24) - flat[pos]            # lands on 2^24 after the add
    cases.append(("reaches 2^24", over))
    for name, dst0 in cases:
        ref = dst0.copy()
        O.flatten(srcs, segs, ref, accumulate=True)
        for f32_decide in (True, False):
            dst = torch.from_numpy(dst0.copy()).cuda()
            H.log(f"fused f32 accumulate: {name}, partials={count}, decide_f32={f32_decide}")
            Z.zero_flatten_norm_bucket_f32(arr, k, dst, partials, n, True)
            Z.zero_step_state_init(st, 1.0)
            if f32_decide:
                Z.zero_shard_decide_f32(partials, count, dst, n, Z.hparams(), st, ws)
            else:
                Z.zero_shard_decide(partials, count, Z.hparams(), st, ws)
            s = Z.read_state(st)
            assert np.array_equal(dst.cpu().numpy().view(np.uint32), ref.view(np.uint32))
            if f32_decide:
                assert _check_sum(s, ref, scale0=1.0) == 0
            else:
                assert (s.wide_pending, s.skip, s.overflow, s.step, s.loss_scale, s.skipped_total) == \
                    (1, 1, 0, 0, 1.0, 0)


def test_accum_skip_and_resume():
    """An inf in one micro-batch poisons the accumulated partition: the step is
    skipped (nothing written, scale halved) and the next one proceeds."""
    w = _small("accum-skip", 50_000, seed=13)
    w.inject = {4: 0x7C00}                        # micro-batch 4 = the first of step 2
    r = H.start_accum(w, 3, fused=True)
    H.step_accum(r)
    snap = [t.clone() for t in (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)]
    H.step_accum(r)
    s = r.dev.read_state()
    assert s.skip == 1 and s.overflow == 1 and s.loss_scale == w.scale0 / 2
    for a, b in zip(snap, (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)):
        assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()
    H.step_accum(r)
    assert r.dev.read_state().step == 2


def test_accum32_periodic_beyond_2_32_elements():
    """Index arithmetic of the accumulation form past 2^32, checked over every
    element: R = 2^20 copies of a K = 4099-element pattern (n = 4,298,113,024,
    77 GB of state).  Two fp16 micro-batches, each from two sources (the first
    read from offset 3 and gathered, the second aligned), are accumulated into
    the fp32 partition in five any-order buckets; the last one's flatten takes
    the exact-norm partials; decision with clipping off; update; two steps.
    The exact sum is the pattern's times 2^20 and S/d, clip off, leaves every
    decision field but the norm the pattern's, so every period of grad32, p32,
    m32, v32 and p16 must equal the oracle's run on the pattern, bit for bit.
    Then an off-grid binary32 pattern written into the partition sends the
    standalone fp32 reduction (1,025 workgroups) to the wide pass over all n
    values, whose rounded sum must be the pattern's exact sum times 2^20."""
    K, R = 4099, 1 << 20
    n = K * R
    a = K << 18
    assert n > (1 << 32) and a % 8 == 0
    segs = [(0, 3, 0, a), (1, 0, a, n - a)]
    S = 1024.0
    rng = np.random.default_rng(96)
    p32 = rng.normal(0.0, 0.02, K).astype(np.float32)
    p16 = shardgen.to_f16_bits(p32)
    m32, v32 = np.zeros(K, np.float32), np.zeros(K, np.float32)
    hp_o, hp_d = O.hparams(max_grad_norm=0.0), Z.hparams(max_grad_norm=0.0)
    st = O.new_state(S)

    def same_as_pattern(d, ref):
        for f in H.STATE_FIELDS:
            assert getattr(d, f) == getattr(ref, f), f
        for f in H.STEP_FIELDS:
            if f not in ("sumsq", "grad_norm"):
                assert np.float64(getattr(d, f)).tobytes() == np.float64(getattr(ref, f)).tobytes(), f
        assert d.sumsq == ref.sumsq * 2.0 ** 20 and d.grad_norm == ref.grad_norm * 2.0 ** 10

    def every_period(t, ref, tdt, ndt):
        return torch.equal(t[:n].view(tdt).view(R, K), torch.from_numpy(ref.view(ndt)).cuda().expand(R, K))

    torch.cuda.empty_cache()
    dev = Z.AccumStep(n, fused=True)
    dev.p32.view(R, K).copy_(torch.from_numpy(p32).cuda().expand(R, K))
    dev.p16.copy_(dev.p32.half())
    dev.init_state(S)
    srcs = [[torch.empty(a + 3, dtype=torch.float16, device="cuda"),
             torch.empty(n - a, dtype=torch.float16, device="cuda")] for _ in range(2)]
    plans = [dev.plan(s, segs, 1 << 30)[1] for s in srcs]
    assert all(len(p) == 5 for p in plans)
    for k in range(2):
        gs = [shardgen.to_f16_bits((rng.normal(0.0, 1e-4, K) * st.loss_scale).astype(np.float32)) for _ in srcs]
        for (sa, sb), g in zip(srcs, gs):
            gd = H.to_dev16(g)
            sa[3:].view(a // K, K).copy_(gd.expand(a // K, K))
            sb.view((n - a) // K, K).copy_(gd.expand((n - a) // K, K))
        H.log(f"accum32 n={n} (period {K}) step {k + 1}: 2 micro-batches")
        dev.step(plans, hp_d)
        grad = np.zeros(K, np.float32)
        for j, g in enumerate(gs):
            O.flatten([g], [(0, 0, 0, K)], grad, accumulate=(j > 0))
        sumsq, ovf = O.norm_overflow_f32(grad)
        O.decide(st, hp_o, sumsq, ovf)
        O.adam_update_f32(st, p16, p32, m32, v32, grad)
        torch.cuda.synchronize()
        same_as_pattern(dev.read_state(), st)
        assert every_period(dev.grad32, grad, torch.int32, np.int32), "grad32"
        for name, ref in (("p32", p32), ("m32", m32), ("v32", v32)):
            assert every_period(getattr(dev, name), ref, torch.int32, np.int32), name
        assert every_period(dev.p16, p16, torch.int16, np.int16), "p16"
        assert dev.guard_intact()

    off = _crafted_f32(K, 97)                           # most values off the 2^-24 grid
    dev.grad32.view(R, K).copy_(torch.from_numpy(off).cuda().expand(R, K))
    st2 = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st2, S)
    assert Z.zero_norm_workspace_bytes(n) >= 1025 * Z.NORM_PARTIAL_BYTES
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    H.log(f"accum32 n={n}: standalone fp32 reduction of an off-grid pattern (wide pass)")
    Z.zero_shard_norm_overflow_f32(dev.grad32, n, hp_d, st2, ws)
    sumsq, ovf = O.norm_overflow_f32(off)
    ref = O.new_state(S)
    O.decide(ref, hp_o, sumsq, ovf)
    d = Z.read_state(st2)
    assert ovf == 0 and d.wide_pending == 0
    same_as_pattern(d, ref)
    del dev, srcs, ws
    torch.cuda.empty_cache()
