"""CPU checks of the C-ABI library: it loads, exports exactly what the header
declares, its host-only functions agree with the oracle, and argument errors
are reported before any device work (so nothing here touches a GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import shardgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_mi355x.h")


@pytest.fixture(scope="module")
def Z():
    from zero_partitioned_mixed_flatten_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    import zero_partitioned_mixed_flatten_amd as Z
    return Z


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(zero_\w+)\s*\(", text, flags=re.M)))


def test_exports_match_header(Z):
    declared = _declared()
    assert declared == sorted(Z.EXPORTS), declared
    L = C.CDLL(Z._lib.LIB_PATH)
    for name in declared:
        assert getattr(L, name) is not None


def test_status_strings(Z):
    for code in (0, -1, -2, -3):
        assert Z.zero_status_string(code)
    assert "unknown" in Z.zero_status_string(-99)


def test_struct_sizes(Z):
    assert C.sizeof(Z.StepState) == 128 and C.sizeof(Z.Segment) == 32 and C.sizeof(Z.HParams) == 80


def test_partial_bytes_match_header(Z):
    # the binding sizes partial buffers with its own copy of the header's constant
    m = re.search(r"#define\s+ZERO_NORM_PARTIAL_BYTES\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == Z.NORM_PARTIAL_BYTES == 16


def test_state_bytes_matches_oracle(Z, oracle):
    rng = np.random.default_rng(5)
    for _ in range(2000):
        psi = int(rng.integers(0, 2 ** 50))
        nd = int(rng.integers(1, 5000))
        k = int(rng.integers(0, 20))
        st = int(rng.integers(0, 4))
        assert Z.zero_state_bytes(psi, nd, k, st) == oracle.state_bytes(psi, nd, k, st)
    assert Z.zero_state_bytes(10 ** 12, 1024, 12, 3) == 15_625_000_000


def test_state_bytes_errors(Z):
    L = Z.lib()
    out = C.c_uint64()
    assert L.zero_state_bytes(10, 0, 12, 3, C.byref(out)) == Z._lib.ZERO_EINVAL
    assert L.zero_state_bytes(10, 1, 12, 5, C.byref(out)) == Z._lib.ZERO_EINVAL
    assert L.zero_state_bytes(10, 1, 12, 3, None) == Z._lib.ZERO_EINVAL
    assert L.zero_state_bytes(2 ** 63, 1, 12, 0, C.byref(out)) == Z._lib.ZERO_ERANGE


@pytest.mark.parametrize("bucket", [1, 7, 1000, 25_000_000])
def test_bucket_segments_cover_exactly(Z, bucket):
    L = shardgen.workload("1t").layout if bucket == 25_000_000 else shardgen.single_tensor_layout(5000)
    if bucket != 25_000_000:
        rng = np.random.default_rng(bucket)
        numels, segs = shardgen.random_segments(rng, 5000, 333)
        L = shardgen.ShardLayout("r", 5000, 1, 0, 0, 5000, ["t"] * len(numels), numels, segs)
    arr, nseg = Z.make_segments([((t + 1) << 40, so, do, c) for t, so, do, c in L.segments])
    pieces = []
    for b in range(0, L.n, bucket):
        out, k = Z.zero_bucket_segments(arr, nseg, b, min(L.n, b + bucket))
        got = [(out[i].src, out[i].src_off, out[i].dst_off, out[i].count) for i in range(k)]
        for src, so, do, c in got:
            assert b <= do and do + c <= min(L.n, b + bucket) and c > 0
        pieces += got
    # the pieces reassemble the original segments exactly
    d = 0
    for src, so, do, c in pieces:
        assert do == d
        d += c
    assert d == L.n
    for t, so, do, c in L.segments:
        mine = [p for p in pieces if p[0] == (t + 1) << 40]
        assert mine[0][1] == so and sum(p[3] for p in mine) == c
        for a, b in zip(mine, mine[1:]):
            assert b[1] == a[1] + a[3]
    if bucket == 25_000_000:
        assert -(-L.n // bucket) == 40


def test_bucket_segments_capacity_error(Z):
    arr, nseg = Z.make_segments([(4096, 0, 0, 10), (8192, 0, 10, 10)])
    L = Z.lib()
    out = (Z.Segment * 1)()
    got = C.c_uint32()
    assert L.zero_bucket_segments(arr, nseg, 0, 20, out, 1, C.byref(got)) == Z._lib.ZERO_ERANGE
    assert got.value == 2
    assert L.zero_bucket_segments(arr, nseg, 5, 4, out, 1, C.byref(got)) == Z._lib.ZERO_EINVAL


def test_workspace_size_is_stable_and_bounded(Z):
    for n in (0, 1, 8, 8191, 1 << 20, 97_350_700, 976_562_500):
        b = Z.zero_norm_workspace_bytes(n)
        assert b == Z.zero_norm_workspace_bytes(n) and 160 <= b <= 512 * 160       # <= 512 wide partials
    assert Z.zero_norm_workspace_bytes(1 << 40) > 512 * 160       # per-thread bound grows the fast grid


# ---- argument validation: every case returns before any device work ---------

FAKE = 1 << 20          # a 16-byte-aligned address that is never dereferenced


@pytest.mark.parametrize("fn", ["zero_shard_adam_step", "zero_shard_adam_step_f32"])
def test_adam_validation(Z, fn):
    L, E = Z.lib(), Z._lib
    ok = dict(p16=FAKE, p32=FAKE, m32=FAKE, v32=FAKE, g=FAKE, st=FAKE)
    call = lambda **kw: getattr(L, fn)(kw["p16"], kw["p32"], kw["m32"], kw["v32"], kw["g"], kw.get("n", 8),
                                       kw["st"], None)
    assert call(**{**ok, "st": 0}) == E.ZERO_EINVAL
    assert call(**{**ok, "p32": 0}) == E.ZERO_EINVAL
    assert call(**{**ok, "m32": FAKE + 4}) == E.ZERO_EALIGN
    assert call(**{**ok, "g": FAKE + 2}) == E.ZERO_EALIGN
    assert call(**{**ok, "g": FAKE + 8}) == E.ZERO_EALIGN
    assert call(**{**ok, "st": FAKE + 4}) == E.ZERO_EALIGN
    assert call(**{**ok, "p16": 0, "n": 0}) == E.ZERO_OK                 # n == 0: nothing to do


def _hp(Z, **kw):
    hp = Z.hparams()
    for k, v in kw.items():
        setattr(hp, k, v)
    return hp


@pytest.mark.parametrize("fn", ["zero_shard_norm_overflow", "zero_shard_norm_overflow_f32"])
def test_norm_validation(Z, fn):
    L, E = Z.lib(), Z._lib
    ws = Z.zero_norm_workspace_bytes(1000)

    def call(hp=None, g=FAKE, n=1000, st=FAKE, w=FAKE, wsb=ws):
        return getattr(L, fn)(g, n, C.byref(hp or Z.hparams()), st, w, wsb, None)

    assert getattr(L, fn)(FAKE, 8, None, FAKE, FAKE, ws, None) == E.ZERO_EINVAL
    assert call(st=0) == E.ZERO_EINVAL and call(w=0) == E.ZERO_EINVAL and call(g=0) == E.ZERO_EINVAL
    for bad in (dict(lr=-1.0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(weight_decay=-1e-3),
                dict(backoff=0.0), dict(backoff=1.5), dict(growth=0.5), dict(min_scale=0.0),
                dict(lr=float("nan")), dict(max_grad_norm=float("inf"))):
        assert call(hp=_hp(Z, **bad)) == E.ZERO_EINVAL, bad
    assert call(g=FAKE + 8) == E.ZERO_EALIGN
    assert call(st=FAKE + 2) == E.ZERO_EALIGN
    assert call(w=FAKE + 8) == E.ZERO_EALIGN
    assert call(wsb=ws - 1) == E.ZERO_ERANGE
    assert call(n=1 << 48, wsb=1 << 40) == E.ZERO_ERANGE


def test_flatten_validation(Z):
    L, E = Z.lib(), Z._lib
    arr, k = Z.make_segments([(FAKE, 0, 0, 100), (FAKE, 0, 100, 100)])
    assert L.zero_flatten_bucket(arr, k, FAKE, 200, 3, 0, None) == E.ZERO_EINVAL          # dtype
    assert L.zero_flatten_bucket(arr, k, 0, 200, E.ZERO_F16, 0, None) == E.ZERO_EINVAL
    assert L.zero_flatten_bucket(arr, k, FAKE + 2, 200, E.ZERO_F16, 0, None) == E.ZERO_EALIGN
    assert L.zero_flatten_bucket(arr, k, FAKE, 199, E.ZERO_F16, 0, None) == E.ZERO_ERANGE
    bad, k2 = Z.make_segments([(FAKE + 1, 0, 0, 10)])
    assert L.zero_flatten_bucket(bad, k2, FAKE, 200, E.ZERO_F16, 0, None) == E.ZERO_EALIGN
    nul, k3 = Z.make_segments([(0, 0, 0, 10)])
    assert L.zero_flatten_bucket(nul, k3, FAKE, 200, E.ZERO_F16, 0, None) == E.ZERO_EINVAL
    assert L.zero_flatten_bucket(None, 0, 0, 0, E.ZERO_F16, 0, None) == E.ZERO_OK


def test_state_init_and_copy_validation(Z):
    L, E = Z.lib(), Z._lib
    assert L.zero_step_state_init(0, 1.0, None) == E.ZERO_EINVAL
    assert L.zero_step_state_init(FAKE, 0.0, None) == E.ZERO_EINVAL
    assert L.zero_step_state_init(FAKE, float("inf"), None) == E.ZERO_EINVAL
    assert L.zero_step_state_init(FAKE + 4, 1.0, None) == E.ZERO_EALIGN
    assert L.zero_stream_copy(0, FAKE, 16, None) == E.ZERO_EINVAL
    assert L.zero_stream_copy(FAKE, FAKE, 15, None) == E.ZERO_EALIGN


def test_flatten_norm_partial_count(Z):
    rng = np.random.default_rng(8)
    numels, segs = shardgen.random_segments(rng, 50_000, 9000)
    arr, k = Z.make_segments([(FAKE, so, do, c) for _, so, do, c in segs] + [(FAKE, 0, 0, 0)])
    want = 0
    for _, _, do, c in segs:                      # one workgroup per 768 aligned 8-vectors, at least one
        head = min((8 - do % 8) % 8, c)
        nv = (c - head) // 8
        want += -(-nv // 768) if nv else 1
    assert Z.zero_flatten_norm_partials(arr, k) == want          # the empty segment needs none
    assert Z.lib().zero_flatten_norm_partials(None, 3) == 0


@pytest.mark.parametrize("fn", ["zero_flatten_norm_bucket", "zero_flatten_norm_bucket_f32"])
def test_fused_validation(Z, fn):
    L, E = Z.lib(), Z._lib
    f = getattr(L, fn)
    arr, k = Z.make_segments([(FAKE, 0, 0, 5000)])
    need = Z.zero_flatten_norm_partials(arr, k)
    assert f(arr, k, FAKE, 5000, 0, 0, need, None) == E.ZERO_EINVAL
    assert f(arr, k, FAKE, 5000, 0, FAKE + 8, need, None) == E.ZERO_EALIGN
    assert f(arr, k, FAKE, 5000, 0, FAKE, need - 1, None) == E.ZERO_ERANGE
    assert f(arr, k, FAKE, 4999, 0, FAKE, need, None) == E.ZERO_ERANGE
    assert f(arr, k, FAKE + 2, 5000, 0, FAKE, need, None) == E.ZERO_EALIGN
    assert f(arr, k, FAKE + 8, 5000, 1, FAKE, need, None) == E.ZERO_EALIGN
    assert f(None, 0, 0, 0, 0, 0, 0, None) == E.ZERO_OK


def test_buckets_validation(Z):
    """zero_flatten_buckets rejects, before any device work, what the
    per-bucket calls reject and also destination ranges that overlap across
    (or within) buckets, since its later launches are not ordered."""
    L, E = Z.lib(), Z._lib
    plan = Z.BucketPlan([Z.make_segments([(FAKE, 0, 0, 3000), (FAKE, 0, 3000, 1000)]),
                         Z.make_segments([(FAKE, 0, 4000, 1000)])])
    need = plan.partials()
    assert need == sum(Z.zero_flatten_norm_partials(a, k) for a, k in plan) == 3
    f = L.zero_flatten_buckets
    call = lambda p=plan, nb=None, dst=FAKE, n=5000, dt=Z.ZERO_F16, acc=0, part=FAKE, cap=need: f(
        p.segs, p.counts, len(p) if nb is None else nb, dst, n, dt, acc, part, cap, None)
    assert call(dt=7) == E.ZERO_EINVAL
    assert f(plan.segs, None, 2, FAKE, 5000, Z.ZERO_F16, 0, 0, 0, None) == E.ZERO_EINVAL
    assert call(n=4999) == E.ZERO_ERANGE
    assert call(dst=FAKE + 2) == E.ZERO_EALIGN
    assert call(part=FAKE + 8) == E.ZERO_EALIGN
    assert call(cap=need - 1) == E.ZERO_ERANGE
    assert call(dt=Z.ZERO_F32, cap=need - 1) == E.ZERO_ERANGE
    for a, b in [((0, 3000), (2999, 10)), ((100, 10), (100, 1)), ((0, 5000), (4000, 1000))]:
        bad = Z.BucketPlan([Z.make_segments([(FAKE, 0, a[0], a[1])]), Z.make_segments([(FAKE, 0, b[0], b[1])])])
        assert f(bad.segs, bad.counts, 2, FAKE, 5000, Z.ZERO_F16, 0, 0, 0, None) == E.ZERO_EINVAL, (a, b)
        assert f(bad.segs, bad.counts, 2, FAKE, 5000, Z.ZERO_F16, 0, FAKE, 1 << 20, None) == E.ZERO_EINVAL
    touching = Z.BucketPlan([Z.make_segments([(FAKE, 0, 0, 3000), (FAKE, 0, 3000, 0), (FAKE, 0, 1000, 0)])])
    assert L.zero_flatten_norm_partials(touching.segs, touching.nsegs) == 1     # empty segments are skipped
    assert f(None, None, 0, 0, 0, Z.ZERO_F16, 0, 0, 0, None) == E.ZERO_OK        # nothing to do


def test_decide_validation(Z):
    L, E = Z.lib(), Z._lib
    ws = Z.zero_decide_workspace_bytes(1000)
    hp = Z.hparams()
    assert L.zero_shard_decide(0, 10, C.byref(hp), FAKE, FAKE, ws, None) == E.ZERO_EINVAL
    assert L.zero_shard_decide(FAKE + 8, 10, C.byref(hp), FAKE, FAKE, ws, None) == E.ZERO_EALIGN
    assert L.zero_shard_decide(FAKE, 1000, C.byref(hp), FAKE, FAKE, 0, None) == E.ZERO_ERANGE
    assert L.zero_shard_decide(FAKE, (1 << 30) + 1, C.byref(hp), FAKE, FAKE, 1 << 20, None) == E.ZERO_ERANGE
    bad = Z.hparams(beta2=1.0)
    assert L.zero_shard_decide(FAKE, 10, C.byref(bad), FAKE, FAKE, ws, None) == E.ZERO_EINVAL


def test_decide_f32_validation(Z):
    L, E = Z.lib(), Z._lib
    ws = Z.zero_decide_workspace_bytes(100)
    hp = Z.hparams()
    call = lambda p=FAKE, c=100, g=FAKE, n=1000, h=C.byref(hp), st=FAKE, w=FAKE, wb=ws: L.zero_shard_decide_f32(
        p, c, g, n, h, st, w, wb, None)
    assert call(g=0) == E.ZERO_EINVAL and call(h=None) == E.ZERO_EINVAL and call(st=0) == E.ZERO_EINVAL
    assert call(g=FAKE + 2) == E.ZERO_EALIGN and call(p=FAKE + 8) == E.ZERO_EALIGN
    assert call(wb=ws - 1) == E.ZERO_ERANGE
    assert call(n=(1 << 40) + 1, wb=1 << 62) == E.ZERO_ERANGE
    assert ws >= 512 * 160                                          # room for the wide pass at any n


def test_onebit_validation(Z):
    L, E = Z.lib(), Z._lib
    n = 1000
    ws = Z.zero_onebit_workspace_bytes(n)
    assert ws > 0 and Z.zero_onebit_workspace_bytes(n) == ws
    ok = [FAKE] * 7
    call = lambda ptrs=ok, nn=n, bw=FAKE, bs=FAKE, st=FAKE, ob=FAKE, wu=2, w=FAKE, wb=ws: L.zero_onebit_step(
        *ptrs, nn, bw, bs, st, ob, wu, w, wb, None)
    assert call(st=0) == E.ZERO_EINVAL and call(ob=0) == E.ZERO_EINVAL and call(w=0) == E.ZERO_EINVAL
    assert call(wu=-1) == E.ZERO_EINVAL
    assert call(bw=0) == E.ZERO_EINVAL
    assert call(ptrs=[FAKE] * 6 + [0]) == E.ZERO_EINVAL
    assert call(ptrs=[FAKE + 8] + [FAKE] * 6) == E.ZERO_EALIGN
    assert call(w=FAKE + 16) == E.ZERO_EALIGN
    assert call(ob=FAKE + 4) == E.ZERO_EALIGN
    assert call(wb=ws - 1) == E.ZERO_ERANGE
    assert call(nn=(1 << 40) + 8, wb=1 << 62) == E.ZERO_ERANGE
    assert L.zero_onebit_state_init(0, None) == E.ZERO_EINVAL
    assert L.zero_onebit_state_init(FAKE + 4, None) == E.ZERO_EALIGN
    assert C.sizeof(Z.OneBitState) == 72


def test_buckets_overlap_check_against_pairwise_model(Z):
    """The multi-bucket call's overlap check (sorted by start, neighbours
    compared) against a brute-force pairwise model on random segment sets cut
    into random buckets: any two nonempty segments sharing a destination
    element -> ZERO_EINVAL; a segment past the destination -> ZERO_ERANGE
    (the range check runs first).  Only sets that must be rejected are
    passed, so nothing is launched."""
    from hypothesis import HealthCheck, given, settings, strategies as hs
    L, E = Z.lib(), Z._lib

    def overlaps(segs):
        live = [(d, d + c) for d, c in segs if c]
        return any(a0 < b1 and b0 < a1 for i, (a0, a1) in enumerate(live) for b0, b1 in live[i + 1:])

    @settings(max_examples=300, deadline=None, suppress_health_check=list(HealthCheck))
    @given(hs.lists(hs.tuples(hs.integers(0, 300), hs.integers(0, 40)), min_size=1, max_size=12),
           hs.integers(1, 4), hs.integers(0, 2 ** 32 - 1))
    def check(segs, nbuckets, cut_seed):
        n = 256
        if not overlaps(segs) and all(d + c <= n for d, c in segs if c):
            return                                           # a valid set would launch: not here
        rng = np.random.default_rng(cut_seed)
        cuts = np.sort(rng.integers(0, len(segs) + 1, nbuckets - 1))
        counts = np.diff(np.concatenate([[0], cuts, [len(segs)]])).astype(np.uint32)
        arr, k = Z.make_segments([(FAKE, 0, d, c) for d, c in segs])
        assert k == len(segs) == int(counts.sum())
        cnt = (C.c_uint32 * len(counts))(*counts.tolist())
        want = E.ZERO_ERANGE if any(d + c > n for d, c in segs if c) else E.ZERO_EINVAL
        for part in (0, FAKE):
            rc = L.zero_flatten_buckets(arr, cnt, len(counts), FAKE, n, Z.ZERO_F16, 0, part, 1 << 20, None)
            assert rc == want, (segs, counts.tolist(), rc, want)

    check()
