"""GPU parity tests of 1-bit Adam on the shard (warm-up with the ordinary fused
step, then the compression stage with frozen variance): the HIP path through
the C ABI against the oracle on the same seeded inputs.

Contract, every step: the step state bitwise; in the compression stage both
scales and their exact sums of squares bitwise, both sign-bit payloads
bitwise, the momentum, both error buffers, p32 and p16 bitwise over the
whole shard (every operation is one binary32 operation in the same order on
both sides, and the scales come from exact sums), and v32 unchanged."""
import numpy as np
import pytest
import torch

import oracle as O
import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _small(name, n, seed, max_seg=None):
    w = shardgen.workload("tiny")
    w.name = name
    rng = np.random.default_rng(seed)
    numels, segs = shardgen.random_segments(rng, n, max_seg or max(1, n // 5))
    w.layout = shardgen.ShardLayout(name, n, 1, 0, 0, n, [f"t{i}" for i in range(len(numels))], numels, segs)
    return w


def _f32(t):
    return t.detach().cpu().numpy().view(np.uint32)


class OneBitRun:
    def __init__(self, w, warmup):
        self.w = w
        n = w.n
        p32 = shardgen.master_params(w)
        self.dev = Z.OneBitStep(n, warmup)
        if n:
            self.dev.p32.copy_(torch.from_numpy(p32))
            self.dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
        self.dev.init_state(w.scale0)
        self.st = O.new_state(w.scale0)
        self.hp_o = H.oracle_hparams(w.hp)
        self.hp_d = H.device_hparams(w.hp)
        z = lambda: np.zeros(n, np.float32)
        self.p32, self.m32, self.v32, self.ew, self.es = p32.copy(), z(), z(), z(), z()
        self.p16 = shardgen.to_f16_bits(p32)
        self.warmup = warmup
        self.k = 0
        self.compressed = 0

    def step(self):
        self.k += 1
        w = self.w
        gpart = shardgen.grad_partition(w, self.k, self.st.loss_scale)
        srcs = shardgen.source_tensors(w.layout, gpart)
        del gpart
        dsrcs = [H.to_dev16(s) for s in srcs]
        compress = self.st.step >= self.warmup
        assert compress == self.dev.compressing()
        H.log(f"onebit {w.name} n={w.n} step {self.k} compress={compress}")
        self.dev.set_segments(dsrcs, w.layout.segments, w.bucket_elems)
        v_before = self.dev.v32.clone()
        self.dev.step(self.hp_d)
        grad = np.empty(w.n, np.uint16)
        O.flatten(srcs, w.layout.segments, grad)
        s, o = O.norm_overflow(grad)
        O.decide(self.st, self.hp_o, s, o)
        if compress:
            bw, bs, (sw, ss) = O.onebit_step(self.st, self.p16, self.p32, self.m32, self.v32, self.ew, self.es, grad)
        else:
            O.adam_update(self.st, self.p16, self.p32, self.m32, self.v32, grad)
        torch.cuda.synchronize()
        H.compare_state(self.dev.read_state(), self.st, None)
        n = w.n
        if compress and not self.st.skip:
            self.compressed += 1
            ob = self.dev.read_onebit()
            assert (ob.scale_w, ob.scale_s) == (np.float32(sw), np.float32(ss)), (ob.scale_w, sw, ob.scale_s, ss)
            assert np.array_equal(self.dev.bits_w.cpu().numpy()[:(n + 7) // 8], bw)
            assert np.array_equal(self.dev.bits_s.cpu().numpy()[:(n + 7) // 8], bs)
            assert torch.equal(self.dev.v32, v_before)                    # frozen
        for name, t, ref in (("p32", self.dev.p32, self.p32), ("m32", self.dev.m32, self.m32),
                             ("v32", self.dev.v32, self.v32), ("err_w", self.dev.err_w, self.ew),
                             ("err_s", self.dev.err_s, self.es)):
            got = _f32(t)[:n]
            assert np.array_equal(got, ref.view(np.uint32)), (name, int(np.sum(got != ref.view(np.uint32))))
        assert np.array_equal(H.bits16(self.dev.p16)[:n], self.p16)
        assert self.dev.guard_intact(), "a kernel stored outside the shard's arrays (arena canary changed)"
        del dsrcs


def test_onebit_tiny_warmup_then_compression():
    r = OneBitRun(shardgen.workload("tiny"), warmup=3)
    for _ in range(8):
        r.step()
    assert r.compressed == 5


@pytest.mark.parametrize("n", [1, 7, 9, 4099, 65_536 * 3 + 5, (1 << 20) + 3, 1 << 22, (1 << 22) + 1])
def test_onebit_ragged(n):
    """Ragged sizes; 2^22 and 2^22 + 1 put the scale folds on either side of
    one workgroup (2048 and 2049 per-workgroup window sums)."""
    r = OneBitRun(_small(f"onebit{n}", n, seed=500 + n), warmup=1)
    for _ in range(3):
        r.step()


def test_onebit_empty():
    w = _small("onebit-empty", 0, seed=0)
    w.layout = shardgen.ShardLayout("empty", 0, 1, 0, 0, 0, [], [], [])
    r = OneBitRun(w, warmup=0)
    r.step()
    ob = r.dev.read_onebit()
    assert (ob.scale_w, ob.scale_s) == (0.0, 0.0)


def test_onebit_gpt2_shard_full_size():
    r = OneBitRun(shardgen.workload("gpt2"), warmup=2)
    for _ in range(4):
        r.step()
    assert r.compressed == 2


def test_onebit_skip_in_compression_stage():
    w = _small("onebit-skip", 100_003, seed=31)
    w.inject = {4: 0x7C00}
    r = OneBitRun(w, warmup=2)
    for _ in range(3):
        r.step()
    snap = [t.clone() for t in (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.err_w, r.dev.err_s)]
    r.step()                                           # step 4: inf -> skipped
    assert r.dev.read_state().skip == 1
    for a, b in zip(snap, (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.err_w, r.dev.err_s)):
        assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()
    r.step()
    assert r.dev.read_state().step == 4


def _crafted(n, seed, lo, hi):
    rng = np.random.default_rng(seed)
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    x = (mant * np.exp2(rng.integers(lo, hi, n).astype(np.float64))).astype(np.float32)
    return x * np.where(rng.integers(0, 2, n) == 1, -1, 1).astype(np.float32)


@pytest.mark.parametrize("case", ["wide", "subnormal", "zeros", "huge", "tie", "span"])
def test_onebit_window_extremes(case):
    """One compression step from crafted momentum and error buffers: values
    spanning 40 binades, binary32 subnormals, all-zero vectors (scale 0, with
    -0.0 entries), magnitudes near 2^100; a worker vector whose sum of
    squares is a binary64 tie broken only by a square 2^-120 below the
    largest (the window cannot round it, the wide pass must); and one whose
    squares span from 2^-298 to 2^200."""
    n = 40_009
    rng = np.random.default_rng({"wide": 11, "subnormal": 12, "zeros": 13, "huge": 14, "tie": 15, "span": 16}[case])
    if case == "wide":
        m, ew, es = (_crafted(n, s, -60, -20) for s in (1, 2, 3))
    elif case == "subnormal":
        m, ew, es = (_crafted(n, s, -170, -140) for s in (4, 5, 6))
    elif case == "zeros":
        m = np.zeros(n, np.float32)
        m[::3] = -0.0
        ew, es = m.copy(), m.copy()
    elif case == "tie":
        m, es = np.zeros(n, np.float32), np.zeros(n, np.float32)
        ew = np.zeros(n, np.float32)                   # x = 0 * beta1 + ew = ew
        ew[[0, 7, 1000, n - 1]] = [1.0, 2.0 ** -27, -(2.0 ** -27), 2.0 ** -60]
    elif case == "span":
        m, es = np.zeros(n, np.float32), _crafted(n, 17, -20, 0)
        ew = _crafted(n, 18, -172, 101)
    else:
        m, ew, es = (_crafted(n, s, 80, 100) for s in (7, 8, 9))
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v32 = (np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32)
    g16 = np.zeros(n, np.uint16)                       # zero gradient: m = beta1 * m
    dev = Z.OneBitStep(n, warmup=0)
    for t, a in ((dev.p32, p32), (dev.m32, m), (dev.v32, v32), (dev.err_w, ew), (dev.err_s, es)):
        t.copy_(torch.from_numpy(a))
    dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
    dev.grad16.copy_(torch.from_numpy(g16.view(np.float16)))
    dev.init_state(1.0)
    hp = Z.hparams(max_grad_norm=0.0)
    Z.zero_shard_norm_overflow(dev.grad16, n, hp, dev.state, dev.workspace)
    H.log(f"onebit window case {case}")
    dev.update()
    st = O.new_state(1.0)
    O.decide(st, O.hparams(max_grad_norm=0.0), *O.norm_overflow(g16))
    refs = [shardgen.to_f16_bits(p32), p32.copy(), m.copy(), v32.copy(), ew.copy(), es.copy()]
    x_w = (np.float32(st.beta1) * m + np.float32(st.omb1) * np.float32(0.0)) + ew   # the worker's input
    bw, bs, (sw, ss) = O.onebit_step(st, *refs, g16)
    torch.cuda.synchronize()
    ob = dev.read_onebit()
    _, S = O.onebit_scale(x_w)
    if case == "tie":
        assert S == 1.0 + 2.0 ** -52                    # the tie broken upward
    assert (ob.scale_w, ob.scale_s) == (np.float32(sw), np.float32(ss))
    assert ob.sumsq_w == S and ob.wide_pending == 0
    assert np.array_equal(dev.bits_w.cpu().numpy(), bw) and np.array_equal(dev.bits_s.cpu().numpy(), bs)
    for t, ref in ((dev.p32, refs[1]), (dev.m32, refs[2]), (dev.err_w, refs[4]), (dev.err_s, refs[5])):
        assert np.array_equal(_f32(t), ref.view(np.uint32))
    assert np.array_equal(H.bits16(dev.p16), refs[0])


@pytest.mark.parametrize("case", ["inf", "nan"])
def test_onebit_non_finite_vector(case):
    """A worker vector holding an inf (or also a NaN), as binary32 overflow
    in the stage's own adds would leave it: both scales are what IEEE
    arithmetic over the squares gives (+inf, or NaN), and everything after
    follows the same binary32 operations as the oracle's.  NaN results may
    differ in their bits (sign and payload are unspecified), so arrays are
    compared with NaN matching NaN."""
    from floatcmp import same_floats32
    n = 10_007
    rng = np.random.default_rng(77)
    m = np.zeros(n, np.float32)
    ew = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    ew[1234] = np.inf
    if case == "nan":
        ew[9000] = np.nan
    es = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    p32 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v32 = (np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32)
    g16 = np.zeros(n, np.uint16)
    dev = Z.OneBitStep(n, warmup=0)
    for t, a in ((dev.p32, p32), (dev.m32, m), (dev.v32, v32), (dev.err_w, ew), (dev.err_s, es)):
        t.copy_(torch.from_numpy(a))
    dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
    dev.grad16.copy_(torch.from_numpy(g16.view(np.float16)))
    dev.init_state(1.0)
    Z.zero_shard_norm_overflow(dev.grad16, n, Z.hparams(max_grad_norm=0.0), dev.state, dev.workspace)
    H.log(f"onebit non-finite vector: {case}")
    dev.update()
    st = O.new_state(1.0)
    O.decide(st, O.hparams(max_grad_norm=0.0), *O.norm_overflow(g16))
    refs = [shardgen.to_f16_bits(p32), p32.copy(), m.copy(), v32.copy(), ew.copy(), es.copy()]
    bw, bs, (sw, ss) = O.onebit_step(st, *refs, g16)
    torch.cuda.synchronize()
    ob = dev.read_onebit()
    want = np.array([sw, ss], np.float32)
    assert same_floats32(np.array([ob.scale_w, ob.scale_s], np.float32), want), (ob.scale_w, ob.scale_s, sw, ss)
    assert (np.isnan(sw) if case == "nan" else sw == np.inf) and ob.wide_pending == 0
    assert np.array_equal(dev.bits_w.cpu().numpy(), bw) and np.array_equal(dev.bits_s.cpu().numpy(), bs)
    for t, ref in ((dev.p32, refs[1]), (dev.m32, refs[2]), (dev.err_w, refs[4]), (dev.err_s, refs[5])):
        assert same_floats32(t.cpu().numpy(), ref)
    got16, want16 = H.bits16(dev.p16), refs[0]
    nan16 = lambda b: ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    assert np.array_equal(nan16(got16), nan16(want16))
    assert np.array_equal(got16[~nan16(got16)], want16[~nan16(want16)])




def test_onebit_periodic_beyond_2_32_elements():
    """Index arithmetic of the 1-bit stage past 2^32, checked over every
    element: the shard is R = 2^20 copies of a K = 4099-element pattern
    (n = 4,298,113,024, 104 GB of state), its gradient flattened in five
    any-order buckets from two sources -- the first read from offset 3, so
    gathered, the second aligned, so the vector path crosses 2^32.  With
    clipping off, every decision field but the norm is the pattern's, the
    exact sums of squares are the pattern's times 2^20 exactly, and S/d is the
    pattern's quotient, so the scales are the pattern's too: every period of
    p32, m32, v32, both error buffers, p16 and both sign payloads must equal
    the oracle's run on the K-element pattern, bit for bit; sumsq and the norm
    are the pattern's times 2^20 and 2^10.  One warm-up step, then two
    compression steps."""
    K, R = 4099, 1 << 20
    n = K * R
    a = K << 18                                      # a multiple of 8 and of K
    assert n > (1 << 32) and n % 8 == 0 and a % 8 == 0
    segs = [(0, 3, 0, a), (1, 0, a, n - a)]
    S = 65536.0
    rng = np.random.default_rng(95)
    p32 = rng.normal(0.0, 0.02, K).astype(np.float32)
    p16 = shardgen.to_f16_bits(p32)
    m32, v32, ew, es = (np.zeros(K, np.float32) for _ in range(4))
    hp_o, hp_d = O.hparams(max_grad_norm=0.0), Z.hparams(max_grad_norm=0.0)
    st = O.new_state(S)

    torch.cuda.empty_cache()
    dev = Z.OneBitStep(n, warmup=1)
    dev.p32.view(R, K).copy_(torch.from_numpy(p32).cuda().expand(R, K))
    dev.p16.copy_(dev.p32.half())
    dev.init_state(S)
    src_a = torch.empty(a + 3, dtype=torch.float16, device="cuda")
    src_b = torch.empty(n - a, dtype=torch.float16, device="cuda")
    shifts = torch.arange(8, dtype=torch.uint8, device="cuda")

    def every_period(t, ref, tdt, ndt):
        """All R periods of t's first n elements equal ref, bit for bit."""
        return torch.equal(t[:n].view(tdt).view(R, K), torch.from_numpy(ref.view(ndt)).cuda().expand(R, K))

    for k in range(3):
        g = shardgen.to_f16_bits((rng.normal(0.0, 1e-4, K) * st.loss_scale).astype(np.float32))
        gd = H.to_dev16(g)
        src_a[3:].view(a // K, K).copy_(gd.expand(a // K, K))
        src_b.view((n - a) // K, K).copy_(gd.expand((n - a) // K, K))
        if k == 0:
            dev.set_segments([src_a, src_b], segs, 1 << 30)
            assert len(dev.buckets) == 5
        compress = st.step >= 1
        H.log(f"onebit n={n} (period {K}) step {k + 1} compress={compress}")
        dev.step(hp_d)
        s, o = O.norm_overflow(g)
        O.decide(st, hp_o, s, o)
        if compress:
            bw, bs, (sw, ss) = O.onebit_step(st, p16, p32, m32, v32, ew, es, g)
        else:
            O.adam_update(st, p16, p32, m32, v32, g)
        torch.cuda.synchronize()
        d = dev.read_state()
        for f in H.STATE_FIELDS:
            assert getattr(d, f) == getattr(st, f), f
        for f in H.STEP_FIELDS:
            if f not in ("sumsq", "grad_norm"):
                assert np.float64(getattr(d, f)).tobytes() == np.float64(getattr(st, f)).tobytes(), f
        assert d.sumsq == st.sumsq * 2.0 ** 20 and d.grad_norm == st.grad_norm * 2.0 ** 10
        for name, ref in (("p32", p32), ("m32", m32), ("v32", v32), ("err_w", ew), ("err_s", es)):
            assert every_period(getattr(dev, name), ref, torch.int32, np.int32), name
        assert every_period(dev.p16, p16, torch.int16, np.int16), "p16"
        if compress:
            ob = dev.read_onebit()
            assert (ob.scale_w, ob.scale_s) == (np.float32(sw), np.float32(ss))
            for name, ref in (("bits_w", bw), ("bits_s", bs)):
                got = ((getattr(dev, name)[:n // 8].unsqueeze(1) >> shifts) & 1).view(R, K)
                want = torch.from_numpy(np.unpackbits(ref, bitorder="little")[:K]).cuda().expand(R, K)
                assert torch.equal(got, want), name
        assert dev.guard_intact()
    del dev, src_a, src_b
    torch.cuda.empty_cache()
