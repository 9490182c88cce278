"""GPU parity tests: the HIP path through the C ABI against the CPU oracle on
the same seeded inputs (contract in tests/gpu_harness.py).

Small and ragged shards are compared element by element over every element;
the full-size shards of the five workloads are compared on sampled elements
(plus every segment boundary and both ends of the shard), with the flattened
gradient, the step state and the fp16 copy checked over the whole shard."""
import numpy as np
import pytest
import torch

import oracle as O
import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402  (tests/ is on sys.path under pytest)
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.float16 else t.view(torch.int32)


def _small(name, n, seed, max_seg=None, misalign=True):
    w = shardgen.workload("tiny")
    w.name = name
    rng = np.random.default_rng(seed)
    numels, segs = shardgen.random_segments(rng, n, max_seg or max(1, n // 5), misalign)
    w.layout = shardgen.ShardLayout(name, n, 1, 0, 0, n, [f"t{i}" for i in range(len(numels))], numels, segs)
    return w


@pytest.mark.parametrize("fused", [False, True])
def test_tiny_workload_ten_steps_full_parity(fused):
    w = shardgen.workload("tiny")
    r = H.start(w, fused=fused)
    for _ in range(w.steps):
        H.step(r)
    assert r.st.step == 10 and r.stats["fp32_not_bitwise"] == 0, r.stats
    H.log(f"tiny: {r.stats}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("n", [1, 7, 8, 9, 63, 4099, 65_536 * 3 + 5, (1 << 20) + 3])
def test_ragged_sizes_misaligned_segments(n, fused):
    w = _small(f"ragged{n}", n, seed=n)
    r = H.start(w, fused=fused)
    for _ in range(3):
        H.step(r)
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.parametrize("blocks", [1, 511, 512, 513, 1024])
def test_decide_around_the_one_wave_fold(blocks):
    """The decide folds up to 512 partials in one wave and more in a
    workgroup: one aligned segment of exactly `blocks` fused-flatten
    workgroups (6144 elements each), stepped against the oracle, with an
    overflow on the third step (the skip path through the same fold)."""
    n = blocks * 6144
    w = _small(f"decide{blocks}", n, seed=blocks)
    w.layout = shardgen.single_tensor_layout(n)
    w.inject = {3: shardgen.F16_POS_INF}
    r = H.start(w, fused=True)
    for _ in range(4):
        H.step(r)
    assert r.dev.partial_count == blocks
    assert r.st.skipped_total == 1 and r.stats["fp32_not_bitwise"] == 0, r.stats



@pytest.mark.parametrize("blocks", [1 << 15, (1 << 15) + 1])
def test_decide_around_the_single_workgroup_limit(blocks):
    """Up to 2^15 partials one workgroup folds them and decides with no
    arrival counter; one more and the fold spreads over several workgroups
    that meet at one.  One aligned segment of exactly `blocks` fused-flatten
    workgroups, 0.5 everywhere but at planted positions (closed-form exact
    sum); two decisions in a row (the counter re-arms), each against the
    oracle bit for bit with the 128-bit sum, and equal, byte for byte, to the
    standalone reduction's over the same partition."""
    from fractions import Fraction
    n = blocks * 6144
    rng = np.random.default_rng(blocks)
    pos = np.unique(np.concatenate([np.array([0, n - 1]), rng.integers(0, n, 40)]))
    bits = (rng.integers(0, 0x7C00, pos.size, dtype=np.uint16)
            | (rng.integers(0, 2, pos.size, dtype=np.uint16) << 15))
    exact = (n - pos.size) * _units16(0x3800) + sum(_units16(int(b)) for b in bits)
    src = torch.full((n,), 0.5, dtype=torch.float16, device="cuda")
    src[torch.from_numpy(pos).cuda()] = H.to_dev16(bits)
    dev = Z.ShardStep(n, fused=True)
    dev.set_segments([src], [(0, 0, 0, n)])
    assert dev.partial_count == blocks
    st2 = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    hp = Z.hparams()
    dev.init_state(65536.0)
    Z.zero_step_state_init(st2, 65536.0)
    ref = O.new_state(65536.0)
    for k in range(2):
        H.log(f"decide over {blocks} partials, call {k + 1}")
        dev.flatten_norm()
        dev.decide(hp)
        Z.zero_shard_norm_overflow(dev.grad16, n, hp, st2, ws)
        O.decide(ref, O.hparams(), float(Fraction(exact, 1 << 48)), 0)
        torch.cuda.synchronize()
        H.compare_state(dev.read_state(), ref, exact)
        assert bytes(dev.state.cpu().numpy()) == bytes(st2.cpu().numpy())



@pytest.mark.parametrize("case", ["never_grow", "no_backoff", "floor", "unit_growth"])
@pytest.mark.parametrize("fused", [False, True])
def test_loss_scaler_edge_settings(case, fused):
    """The dynamic loss scaler at the edges of its settings, stepped against
    the oracle with overflows injected at steps 2, 3 (a NaN), 4 and 9:
    growth_interval 0 (the scale never grows), backoff 1 (an overflow skips
    the step and keeps the scale), a floor above 1 (repeated overflows stop
    at min_scale), growth 1 every clean step (a growth that leaves the scale
    unchanged).  Every state field bitwise each step, and the trajectory the
    setting implies."""
    from dataclasses import replace
    w = _small(f"scaler-{case}", 20_003, seed=60)
    settings = {"never_grow": dict(growth_interval=0), "no_backoff": dict(backoff=1.0),
                "floor": dict(min_scale=2.0 ** 14), "unit_growth": dict(growth=1.0, growth_interval=1)}[case]
    w.hp = replace(w.hp, **settings)
    w.scale0 = 2.0 ** 16
    w.inject = {2: shardgen.F16_POS_INF, 3: shardgen.F16_NAN_SENTINEL, 4: shardgen.F16_POS_INF,
                9: shardgen.F16_POS_INF}
    r = H.start(w, fused=fused)
    scales = []
    for _ in range(12):
        H.step(r)
        scales.append(r.dev.read_state().loss_scale)
    assert r.st.skipped_total == 4 and r.st.step == 8
    want = {"never_grow": 2.0 ** 12, "no_backoff": 2.0 ** 16, "floor": 2.0 ** 14, "unit_growth": 2.0 ** 12}[case]
    assert scales[-1] == want, scales
    if case != "no_backoff":
        assert all(b <= a for a, b in zip(scales, scales[1:])), scales       # never grows


@pytest.mark.parametrize("any_order", [False, True])
@pytest.mark.parametrize("fused", [False, True])
def test_many_segments_over_launch_limit(fused, any_order):
    # > 64 segments forces several flatten launches in one call
    w = _small("many", 300_000, seed=3, max_seg=2000, misalign=False)
    assert len(w.layout.segments) > 64
    r = H.start(w, fused=fused, any_order=any_order)
    for _ in range(2):
        H.step(r)


@pytest.mark.parametrize("fused", [False, True])
def test_empty_shard(fused):
    w = _small("empty", 0, seed=0)
    w.layout = shardgen.ShardLayout("empty", 0, 1, 0, 0, 0, [], [], [])
    r = H.start(w, fused=fused)
    H.step(r)
    s = r.dev.read_state()
    assert s.sumsq == 0.0 and s.step == 1 and s.overflow == 0


def test_gpt2_shard_full_size_separate_path():
    w = shardgen.workload("gpt2")
    r = H.start(w, sample=1 << 20, fused=False)
    for _ in range(3):
        t = H.step(r)
        H.log(f"gpt2 timings {t}")
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.timeout(900)
def test_gpt2_shard_all_100_steps():
    """The GPT-2 1.5B-like workload at its stated length: 100 fused steps on
    the full rank-8 shard, every step's decision and state bitwise, sampled
    elements against the oracle, the whole-shard fp16 cast every 10th step."""
    w = shardgen.workload("gpt2")
    assert w.steps == 100
    r = H.start(w, sample=1 << 16, fused=True)
    for k in range(1, w.steps + 1):
        H.step(r, check_full_cast=(k % 10 == 0), exact=(k % 25 == 0))
    s = r.dev.read_state()
    assert (s.step, s.skipped_total) == (100, 0) and s.loss_scale == 2.0 ** (16 + 5), s.as_dict()
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.timeout(900)
def test_stress_loss_scale_trajectory_full_size():
    w = shardgen.workload("stress")
    r = H.start(w, sample=1 << 16, fused=True)
    snap = None
    for k in range(1, w.steps + 1):
        if k in w.inject:
            snap = [t.clone() for t in (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)]
        H.step(r, check_full_cast=(k % 10 == 0), exact=(k % 25 == 0))
        if k in w.inject:
            s = r.dev.read_state()
            assert s.skip == 1 and s.overflow == 1
            for a, b in zip(snap, (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)):
                assert torch.equal(_bits(a), _bits(b))
            snap = None
    s = r.dev.read_state()
    assert (s.loss_scale, s.good_steps, s.step, s.skipped_total) == (2.0 ** 26, 13, 98, 2)


def test_100b_shard_full_size_separate_path():
    w = shardgen.workload("100b")
    r = H.start(w, sample=1 << 20, fused=False)
    for _ in range(2):
        H.step(r)


@pytest.mark.timeout(900)
def test_100b_shard_all_50_steps_clipping():
    """The 100B workload at its stated length: 50 fused steps on the rank-12
    shard with clipping active on every step (the gradient norm stays above
    1), so the bias corrections ramp through 50 clipped updates."""
    w = shardgen.workload("100b")
    assert w.steps == 50
    r = H.start(w, sample=1 << 16, fused=True)
    for k in range(1, w.steps + 1):
        H.step(r, check_full_cast=(k % 10 == 0), exact=False)
        assert r.st.grad_norm > w.hp.max_grad_norm, (k, r.st.grad_norm)
    s = r.dev.read_state()
    assert (s.step, s.skipped_total) == (50, 0), s.as_dict()
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.timeout(900)
def test_1t_shard_all_20_steps_bucketed():
    """The 1T workload at its stated length: 20 fused steps on the rank-512
    shard, each flattened in 40 bucket calls of 25M elements; the loss scale
    grows at the 20th clean step."""
    w = shardgen.workload("1t")
    assert w.steps == 20
    r = H.start(w, sample=1 << 16, fused=True)
    assert len(r.dev.buckets) == 0
    for k in range(1, w.steps + 1):
        H.step(r, check_full_cast=(k % 10 == 0), exact=False)
        assert len(r.dev.buckets) == 40
    s = r.dev.read_state()
    assert (s.step, s.skipped_total, s.good_steps) == (20, 0, 0) and s.loss_scale == 2.0 ** 17, s.as_dict()
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.parametrize("dtype,acc", [(Z.ZERO_F16, False), (Z.ZERO_F16, True), (Z.ZERO_F32, False),
                                       (Z.ZERO_F32, True)])
def test_flatten_modes(dtype, acc):
    rng = np.random.default_rng(dtype * 10 + acc)
    n = 200_003
    numels, segs = shardgen.random_segments(rng, n, 30_000)
    holes = [s for i, s in enumerate(segs) if i % 4 != 2]           # leave some destination untouched
    srcs = [shardgen.to_f16_bits((rng.standard_normal(k) * 300).astype(np.float32)) for k in numels]
    if dtype == Z.ZERO_F16:
        dst0 = shardgen.to_f16_bits((rng.standard_normal(n) * 300).astype(np.float32))
        dev_dst = H.to_dev16(dst0.copy())
    else:
        dst0 = (rng.standard_normal(n) * 300).astype(np.float32)
        dev_dst = torch.from_numpy(dst0.copy()).cuda()
    ref = dst0.copy()
    O.flatten(srcs, holes, ref, accumulate=acc)
    dsrcs = [H.to_dev16(s) for s in srcs]
    arr, k = Z.make_segments([(dsrcs[t].data_ptr(), so, do, c) for t, so, do, c in holes])
    H.log(f"flatten mode dtype={dtype} acc={acc} segments={k}")
    Z.zero_flatten_bucket(arr, k, dev_dst, n, dtype, acc)
    torch.cuda.synchronize()
    got = dev_dst.cpu().numpy()
    assert np.array_equal(got.view(np.uint16) if dtype == Z.ZERO_F16 else got.view(np.uint32),
                          ref.view(np.uint16) if dtype == Z.ZERO_F16 else ref.view(np.uint32))


def test_fp16_copy_rounding_sweep():
    """lr = wd = 0 and a zero gradient leave p32 unchanged, so p16 = fp16(p32)
    for every finite fp32 pattern of a stratified sweep (all exponents, and
    every low-bit pattern around the binary16 subnormal/normal/overflow
    boundaries), compared with the oracle's own converter."""
    rng = np.random.default_rng(5)
    parts = [(np.repeat(np.arange(255, dtype=np.uint32), 1 << 14) << 23) |
             rng.integers(0, 1 << 23, 255 << 14, dtype=np.uint32)]
    low = np.arange(1 << 15, dtype=np.uint32)
    for e in range(127 - 27, 127 + 17):
        parts.append((np.uint32(e) << np.uint32(23)) | (np.uint32(rng.integers(0, 256)) << np.uint32(15)) | low)
    bits = np.concatenate(parts)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    p = bits.view(np.float32)
    n = p.size
    dev = Z.ShardStep(n)
    dev.p32.copy_(torch.from_numpy(p))
    dev.init_state(1.0)
    hp = Z.hparams(lr=0.0, weight_decay=0.0)
    H.log(f"fp16 sweep n={n}")
    dev.norm_overflow(hp)
    dev.adam()
    torch.cuda.synchronize()
    assert np.array_equal(dev.p32.cpu().numpy().view(np.uint32), bits)
    assert np.array_equal(H.bits16(dev.p16), O.f16_from_f32(p))



@pytest.mark.parametrize("bits", [0x0000, 0x8000])
@pytest.mark.parametrize("fused", [False, True])
def test_all_zero_gradient(bits, fused):
    """A gradient of +0.0 (or -0.0) everywhere, clipping on: the exact sum is
    0, the norm 0 and the clip coefficient 1 (the threshold over a zero norm
    never reaches the state), m and v stay zero and the update is the weight
    decay alone.  Three steps on a ragged shard in three segments; every
    state field, p16 and p32/m32/v32 over the whole shard, bit for bit,
    against the oracle."""
    n = 70_001
    rng = np.random.default_rng(61)
    segs = [(0, 0, 0, 20_000), (1, 3, 20_000, 30_001), (0, 20_000, 50_001, 20_000)]
    g = np.full(n, bits, np.uint16)
    srcs = [np.full(40_000, bits, np.uint16), np.full(30_004, bits, np.uint16)]
    p32 = rng.normal(0.0, 0.02, n).astype(np.float32)
    p16, m32, v32 = shardgen.to_f16_bits(p32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    dev = Z.ShardStep(n, fused=fused)
    dev.p32.copy_(torch.from_numpy(p32))
    dev.p16.copy_(torch.from_numpy(p16.view(np.float16)))
    dev.init_state(65536.0)
    dsrcs = [H.to_dev16(x) for x in srcs]
    dev.set_segments(dsrcs, segs)
    hp_o, hp_d = O.hparams(max_grad_norm=1.0), Z.hparams(max_grad_norm=1.0)
    st = O.new_state(65536.0)
    for k in range(3):
        H.log(f"zero gradient {bits:#06x} fused={fused} step {k + 1}")
        dev.step(hp_d)
        s, o = O.norm_overflow(g)
        assert (s, o) == (0.0, 0)
        O.decide(st, hp_o, s, o)
        O.adam_update(st, p16, p32, m32, v32, g)
        torch.cuda.synchronize()
        H.compare_state(dev.read_state(), st, 0)
        assert np.array_equal(H.bits16(dev.grad16), g)
        assert np.array_equal(H.bits16(dev.p16), p16)
        for name, ref in (("p32", p32), ("m32", m32), ("v32", v32)):
            assert np.array_equal(getattr(dev, name).cpu().numpy().view(np.uint32), ref.view(np.uint32)), name
    assert st.gmul == np.float32(1.0 / 65536.0) and not m32.any() and not v32.any()



def test_two_shards_on_two_streams():
    """Calls on different streams with disjoint buffers may run at once: two
    shards (the fused path in five any-order buckets, and the separate path)
    are prepared first, then enqueued back to back on two streams of default
    priority, so that their kernels overlap on the GPU; three steps, with an
    overflow on the second step of the second shard.  Each matches the
    oracle as if it ran alone (sampled p/m/v, the whole flattened gradient,
    the state and p16 = fp16(p32) over the whole shard)."""
    w1 = _small("streams-a", 24_000_011, seed=81)
    w1.bucket_elems = 5_000_000
    w2 = _small("streams-b", 20_000_003, seed=82)
    w2.inject = {2: shardgen.F16_POS_INF}
    r1 = H.start(w1, sample=1 << 16, fused=True)
    r2 = H.start(w2, sample=1 << 16, fused=False)
    torch.cuda.synchronize()                       # the set-up, on the default stream, is done
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        p1, p2 = H.prepare(r1), H.prepare(r2)
        H.enqueue(r1, p1, s1)
        H.enqueue(r2, p2, s2)
        H.finish(r1, p1)
        H.finish(r2, p2)
    assert r1.st.skipped_total == 0 and r2.st.skipped_total == 1 and r2.st.step == 2
    assert r1.stats["fp32_not_bitwise"] == 0 and r2.stats["fp32_not_bitwise"] == 0


def test_skip_and_resume_bitwise():
    w = _small("resume", 100_000, seed=9)
    w.inject = {2: 0xFC00}
    straight = H.start(w)
    for _ in range(6):
        H.step(straight)
    a = H.start(w)
    for _ in range(3):
        H.step(a)
    saved = [t.cpu() for t in (a.dev.p16, a.dev.p32, a.dev.m32, a.dev.v32, a.dev.state)]
    b = H.start(w)                                  # fresh buffers, then restore
    for t, s in zip((b.dev.p16, b.dev.p32, b.dev.m32, b.dev.v32, b.dev.state), saved):
        t.copy_(s)
    b.st, b.p16, b.p32, b.m32, b.v32, b.k = a.st, a.p16, a.p32, a.m32, a.v32, a.k
    for _ in range(3):
        H.step(b)
    for x, y in zip((straight.dev.p16, straight.dev.p32, straight.dev.m32, straight.dev.v32, straight.dev.state),
                    (b.dev.p16, b.dev.p32, b.dev.m32, b.dev.v32, b.dev.state)):
        assert x.cpu().numpy().tobytes() == y.cpu().numpy().tobytes()
    assert straight.dev.read_state().skipped_total == 1


def test_norm_special_values_everywhere():
    """inf/NaN patterns in the vector body, in the ragged tail and at the
    first element all raise the flag; the largest finite values do not."""
    n = 8 * 5000 + 5
    rng = np.random.default_rng(4)
    base = shardgen.to_f16_bits((rng.standard_normal(n) * 100).astype(np.float32))
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    cases = [(0, 0x7C00), (n - 1, 0xFC00), (n - 3, 0x7E00), (12345, 0x7C01), (8 * 4999, 0xFFFF),
             (None, 0x7BFF)]
    for pos, val in cases:
        g = base.copy()
        if pos is None:
            g[::7] = val
        else:
            g[pos] = val
        Z.zero_step_state_init(st, 1024.0)
        H.log(f"norm special pos={pos} val={val:#x}")
        Z.zero_shard_norm_overflow(H.to_dev16(g), n, Z.hparams(), st, ws)
        s = Z.read_state(st)
        sumsq, ovf = O.norm_overflow(g)
        assert s.overflow == ovf == (1 if pos is not None else 0)
        assert np.float64(s.sumsq).tobytes() == np.float64(sumsq).tobytes()
        if not ovf:
            assert s.as_dict()["sumsq_units"] == H.exact_units(g)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_standalone_norm_multi_workgroup_fold(dtype):
    """The standalone norm over a quarter-billion-element partition: every
    one of its workgroups streams thousands of elements and all of them meet
    at the arrival counter.  The exact sum, the flag and the decision equal
    the oracle's, bit for bit; a second call re-uses the re-armed counter."""
    n = (1 << 28) + 7 * 8192 + 3
    rng = np.random.default_rng(90 if dtype == "f16" else 91)
    g16 = rng.integers(0, 0x7C00, n, dtype=np.uint16) | (rng.integers(0, 2, n, dtype=np.uint16) << 15)
    if dtype == "f16":
        dev = H.to_dev16(g16)
        ref = O.norm_overflow(g16)
        call = Z.zero_shard_norm_overflow
    else:
        g32 = g16.view(np.float16).astype(np.float32) * np.float32(256.0)     # |x| < 2^24, exact
        del g16
        dev = torch.from_numpy(g32).cuda()
        ref = O.norm_overflow_f32(g32)
        call = Z.zero_shard_norm_overflow_f32
        del g32
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st, 65536.0)
    hp_d = Z.hparams()
    ost = O.new_state(65536.0)
    for k in range(2):
        H.log(f"standalone norm {dtype} n={n} call {k}")
        call(dev, n, hp_d, st, ws)
        O.decide(ost, O.hparams(), *ref)
        s = Z.read_state(st)
        assert (s.overflow, np.float64(s.sumsq).tobytes()) == (ref[1], np.float64(ref[0]).tobytes())
        H.compare_state(s, ost, None)


@pytest.mark.parametrize("n,grid", [((1 << 30) + 1, 257), ((1 << 31) + 12345, 513)])
def test_standalone_norm_beyond_256_workgroups(n, grid):
    """Above 2^30 elements the standalone norm's grid grows past one
    workgroup per CU (no thread sums more than 4096 values): 257 workgroups
    at 2^30 + 1 (the last workgroup folds the partials in two batches, the
    second holding one) and 513 at 2^31 + 12,345 (three batches).  The
    partition is one value everywhere but at planted positions, so its exact
    sum is a closed form; the 128-bit sum, its rounding and the decision must
    match it bit for bit."""
    from fractions import Fraction
    rng = np.random.default_rng(92)
    pos = np.unique(rng.integers(0, n, 64))
    bits = rng.integers(0, 0x7C00, pos.size, dtype=np.uint16) | (rng.integers(0, 2, pos.size, dtype=np.uint16) << 15)
    dev = torch.full((n,), 0.5, dtype=torch.float16, device="cuda")
    dev[torch.from_numpy(pos).cuda()] = H.to_dev16(bits)

    def units(b):                                   # x^2 in units of 2^-48 from the binary16 fields
        f, m = (int(b) >> 10) & 31, int(b) & 1023
        e = f - 25 if f else -24
        return (m | (1024 if f else 0)) ** 2 << (2 * e + 48)
    exact = (n - pos.size) * (1 << 46) + sum(units(b) for b in bits)
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    assert Z.zero_norm_workspace_bytes(n) >= grid * Z.NORM_PARTIAL_BYTES
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st, 65536.0)
    ost = O.new_state(65536.0)
    for k in range(2):
        H.log(f"standalone norm n={n} ({grid} workgroups) call {k}")
        Z.zero_shard_norm_overflow(dev, n, Z.hparams(), st, ws)
        O.decide(ost, O.hparams(), float(Fraction(exact, 1 << 48)), 0)
        s = Z.read_state(st)
        assert (int(s.sumsq_units[1]) << 64 | int(s.sumsq_units[0])) == exact and s.overflow == 0
        assert s.sumsq == float(Fraction(exact, 1 << 48))
        H.compare_state(s, ost, None)


def test_fused_flatten_sum_at_the_magnitude_bound():
    """The fused flatten folds each wave's squares in binary64, which stays
    exact while a lane adds at most 46 of them: here every value is +-65504
    (the largest finite binary16, square just below 2^32) over several full
    workgroups and misaligned segments, so the first workgroup of each
    segment adds head and tail elements on top of its vectors, plus a few
    2^-24 subnormals whose 2^-48 squares any rounding at that magnitude would
    lose.  The 128-bit sum equals the closed form, bit for bit, through the
    plain and the bucketed call."""
    rng = np.random.default_rng(93)
    n = 5 * 6144 + 6 * 8 + 5
    numels, segs = shardgen.random_segments(rng, n, 4000, True)
    assert any(do % 8 for _, _, do, _ in segs)                  # some segment heads and tails
    vals = np.where(rng.integers(0, 2, n) == 1, np.uint16(0x7BFF), np.uint16(0xFBFF))
    tiny = rng.choice(n, 9, replace=False)
    vals[tiny] = np.uint16(0x0001)                             # 2^-24: square 2^-48, one unit
    srcs, k = [], 0
    for (t, so, do, c), m in zip(segs, numels):
        buf = rng.integers(0, 0x7C00, m, dtype=np.uint16)      # padding around the segment: not summed
        buf[so:so + c] = vals[do:do + c]
        srcs.append(H.to_dev16(buf))
    arr, kk = Z.make_segments([(srcs[t].data_ptr(), so, do, c) for t, so, do, c in segs])
    exact = (n - tiny.size) * (65504 ** 2 << 48) + tiny.size
    for bucket in (0, 7000):
        plan = [(arr, kk)] if not bucket else [Z.zero_bucket_segments(arr, kk, b, min(n, b + bucket))
                                               for b in range(0, n, bucket)]
        plan = Z.BucketPlan(plan)
        count = plan.partials()
        dst = torch.zeros(n, dtype=torch.float16, device="cuda")
        parts = torch.empty(count * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
        ws = torch.empty(max(16, Z.zero_decide_workspace_bytes(count)), dtype=torch.uint8, device="cuda")
        st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
        Z.zero_step_state_init(st, 1.0)
        H.log(f"fused flatten at the magnitude bound: n={n} buckets={len(plan)}")
        Z.zero_flatten_buckets(plan, dst, n, Z.ZERO_F16, False, parts)
        Z.zero_shard_decide(parts, count, Z.hparams(), st, ws)
        s = Z.read_state(st)
        assert s.overflow == 0 and (int(s.sumsq_units[1]) << 64 | int(s.sumsq_units[0])) == exact
        assert np.array_equal(H.bits16(dst), vals)


def test_determinism_two_runs():
    w = _small("det", 777_777, seed=12)
    outs = []
    for _ in range(2):
        r = H.start(w)
        for _ in range(2):
            H.step(r, check=False)
        torch.cuda.synchronize()
        outs.append(b"".join(t.cpu().numpy().tobytes() for t in (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32,
                                                                r.dev.state)))
    assert outs[0] == outs[1]


def test_stream_copy():
    x = torch.randint(0, 2 ** 31 - 1, ((1 << 22) + 4,), dtype=torch.int32, device="cuda")
    y = torch.zeros_like(x)
    Z.zero_stream_copy(y, x, x.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


def test_fused_and_separate_paths_decide_identically():
    """The fused flatten + decide and the flatten + standalone norm take the
    same decision bit for bit (both sums are exact), and write the same
    partition, on a bucketed layout with misaligned segments."""
    w = _small("fused-vs-separate", 3_000_017, seed=21, max_seg=400_000)
    w.bucket_elems = 1_000_000
    runs = [H.start(w, fused=f) for f in (False, True)]
    for _ in range(3):
        for r in runs:
            H.step(r)
        a, b = (r.dev.read_state() for r in runs)
        assert bytes(a) == bytes(b)
        assert torch.equal(runs[0].dev.grad16.view(torch.int16), runs[1].dev.grad16.view(torch.int16))
    for x, y in zip((runs[0].dev.p16, runs[0].dev.p32), (runs[1].dev.p16, runs[1].dev.p32)):
        assert torch.equal(_bits(x), _bits(y))


def test_fused_flatten_accumulate_norm():
    """Gradient accumulation in fp16: the fused flatten's partials describe the
    accumulated values it stores."""
    rng = np.random.default_rng(33)
    n = 100_003
    numels, segs = shardgen.random_segments(rng, n, 20_000)
    srcs = [shardgen.to_f16_bits((rng.standard_normal(k) * 50).astype(np.float32)) for k in numels]
    dst0 = shardgen.to_f16_bits((rng.standard_normal(n) * 50).astype(np.float32))
    ref = dst0.copy()
    O.flatten(srcs, segs, ref, accumulate=True)
    dsrcs = [H.to_dev16(s) for s in srcs]
    arr, k = Z.make_segments([(dsrcs[t].data_ptr(), so, do, c) for t, so, do, c in segs])
    count = Z.zero_flatten_norm_partials(arr, k)
    partials = torch.empty(count * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = H.to_dev16(dst0.copy())
    H.log(f"fused accumulate n={n} partials={count}")
    Z.zero_flatten_norm_bucket(arr, k, dst, partials, n, True)
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st, 1.0)
    ws = torch.empty(max(16, Z.zero_decide_workspace_bytes(count)), dtype=torch.uint8, device="cuda")
    Z.zero_shard_decide(partials, count, Z.hparams(), st, ws)
    s = Z.read_state(st)
    assert np.array_equal(H.bits16(dst), ref)
    sumsq, ovf = O.norm_overflow(ref)
    assert s.overflow == ovf == 0 and np.float64(s.sumsq).tobytes() == np.float64(sumsq).tobytes()
    assert s.as_dict()["sumsq_units"] == H.exact_units(ref)



def _units16(b: int) -> int:
    """The square of a finite binary16 value, from its fields, in units of 2^-48."""
    f, m = (b >> 10) & 31, b & 1023
    e = f - 25 if f else -24
    return (m | (1024 if f else 0)) ** 2 << (2 * e + 48)


def _where_not(t: torch.Tensor, value: int) -> np.ndarray:
    """Indices of the elements of a 1-D integer tensor that differ from value,
    in chunks of 2^30 (torch's nonzero is limited to 2^31 - 1 elements)."""
    out = [np.zeros(0, np.int64)]
    for lo in range(0, t.numel(), 1 << 30):
        out.append((torch.nonzero(t[lo:lo + (1 << 30)] != value).flatten() + lo).cpu().numpy())
    return np.concatenate(out)


def test_fused_step_beyond_2_32_elements():
    """Index arithmetic past 2^32: a 4,294,970,407-element partition (17.2 GB
    per fp32 array, 69 GB of state in the arena) from three per-layer
    tensors -- the second starting at an odd destination offset, so its body
    is gathered, the third read from source offset 5 -- flattened in 17
    any-order buckets with exact-norm partials, decided from about 700,000
    partials over 256 workgroups with clipping active, and updated; two
    steps.  The gradient is 0.5 and the master parameter 0.0123 everywhere
    but at planted positions (segment and bucket edges, around 2^32, the
    ragged tail, and random ones), so the exact sum is a closed form.
    Checked: the state bit for bit; the flattened partition differs from 0.5
    exactly at the planted positions, with their values; p32/m32/v32/p16 at
    the planted positions and at 2,000 random others equal the oracle's
    update; every element of p32, m32 and v32 outside the planted set equals
    the oracle's update of the common element (so all n were updated);
    p16 = fp16(p32) everywhere; the arena's guards are intact.  Then the
    standalone norm over the same partition (1,025 workgroups) gives the
    same 128-bit sum and decision."""
    from fractions import Fraction
    n = (1 << 32) + 4 * 777 + 3
    a, b = 1_431_656_771, 1_431_655_765               # a odd: the second segment starts misaligned
    c = n - a - b
    segs = [(0, 0, 0, a), (1, 0, a, b), (2, 5, a + b, c)]
    bucket = 1 << 28
    c16, p_common, S = 0x3800, np.float32(0.0123), 65536.0

    rng = np.random.default_rng(94)
    edges = [0, 1, 7, 8, a - 1, a, a + 1, a + b - 1, a + b, a + b + 1, (1 << 32) - 1, 1 << 32, (1 << 32) + 1]
    edges += [k * bucket + d for k in range(1, n // bucket + 1) for d in (-1, 0, 1)]
    edges += list(range(n - 9, n))
    planted = np.unique(np.concatenate([np.array(edges, np.int64), rng.integers(0, n, 300)]))
    g_pl = (rng.integers(0, 0x7C00, planted.size, dtype=np.uint16)
            | (rng.integers(0, 2, planted.size, dtype=np.uint16) << 15))
    g_pl[g_pl == c16] ^= 1                               # every planted value differs from the common one
    p_pl = rng.normal(0.0, 0.05, planted.size).astype(np.float32)
    others = np.setdiff1d(rng.integers(0, n, 2000), planted)
    sample = np.concatenate([planted, others])           # the elements the oracle updates

    torch.cuda.empty_cache()
    srcs = [torch.full((a,), 0.5, dtype=torch.float16, device="cuda"),
            torch.full((b,), 0.5, dtype=torch.float16, device="cuda"),
            torch.full((c + 5,), 0.5, dtype=torch.float16, device="cuda")]
    for t, so, do, cnt in segs:                          # planted through the sources
        sel = (planted >= do) & (planted < do + cnt)
        srcs[t][torch.from_numpy(planted[sel] - do + so).cuda()] = H.to_dev16(g_pl[sel])
    dev = Z.ShardStep(n, fused=True, any_order=True)
    pl_dev = torch.from_numpy(planted).cuda()
    dev.p32.fill_(float(p_common))
    dev.p32[pl_dev] = torch.from_numpy(p_pl).cuda()
    dev.p16.copy_(dev.p32.half())
    dev.init_state(S)
    dev.set_segments(srcs, segs, bucket)
    assert len(dev.buckets) == 17 and dev.partial_count > 600_000

    # the oracle's side: the sampled elements, and the common element alone
    g_s = np.full(sample.size, c16, np.uint16)
    g_s[:planted.size] = g_pl
    p32_s = np.full(sample.size, p_common, np.float32)
    p32_s[:planted.size] = p_pl
    p16_s, m32_s, v32_s = shardgen.to_f16_bits(p32_s), np.zeros_like(p32_s), np.zeros_like(p32_s)
    c_p32 = np.array([p_common], np.float32)
    c_p16, c_m32, c_v32, c_g = shardgen.to_f16_bits(c_p32), np.zeros(1, np.float32), np.zeros(1, np.float32), \
        np.array([c16], np.uint16)
    exact = (n - planted.size) * _units16(c16) + sum(_units16(int(v)) for v in g_pl)
    sumsq = float(Fraction(exact, 1 << 48))
    hp_o, hp_d = O.hparams(max_grad_norm=0.3), Z.hparams(max_grad_norm=0.3)
    ost = O.new_state(S)
    it = torch.from_numpy(sample).cuda()
    for k in range(2):
        H.log(f"fused step n={n} (17 buckets, {dev.partial_count} partials) step {k + 1}")
        dev.step(hp_d)
        O.decide(ost, hp_o, sumsq, 0)
        assert not ost.skip and ost.gmul < 1.0 / S                         # clipping is active
        O.adam_update(ost, p16_s, p32_s, m32_s, v32_s, g_s)
        O.adam_update(ost, c_p16, c_p32, c_m32, c_v32, c_g)
        torch.cuda.synchronize()
        H.compare_state(dev.read_state(), ost, exact)
        assert np.array_equal(H.bits16(dev.p16[it]), p16_s)
        for name, ref in (("p32", p32_s), ("m32", m32_s), ("v32", v32_s)):
            got = getattr(dev, name)[it].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
        if k == 0:
            assert np.array_equal(_where_not(dev.grad16.view(torch.int16), c16), planted), \
                "flattened partition: the positions that differ from the common value are not the planted ones"
            assert np.array_equal(H.bits16(dev.grad16[pl_dev]), g_pl)
    for name, ref in (("p32", c_p32), ("m32", c_m32), ("v32", c_v32)):
        off = _where_not(getattr(dev, name).view(torch.int32), int(ref.view(np.int32)[0]))
        assert np.isin(off, planted).all(), f"{name}: {int((~np.isin(off, planted)).sum())} unplanted elements differ"
    assert torch.equal(dev.p16.view(torch.int16), dev.p32.half().view(torch.int16))
    assert dev.guard_intact()

    st2 = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st2, S)
    assert Z.zero_norm_workspace_bytes(n) >= 1025 * Z.NORM_PARTIAL_BYTES
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    H.log(f"standalone norm over the same partition, n={n}")
    Z.zero_shard_norm_overflow(dev.grad16, n, hp_d, st2, ws)
    ost2 = O.new_state(S)
    O.decide(ost2, hp_o, sumsq, 0)
    H.compare_state(Z.read_state(st2), ost2, exact)
    del srcs, dev, ws, it, pl_dev
    torch.cuda.empty_cache()
