"""zero_flatten_buckets against one ordered call per bucket.

The multi-bucket call issues every launch after its first without the
dispatch barrier, so consecutive buckets run at the same time on the GPU.
Its stores and partials must nevertheless be exactly those of the per-bucket
calls (zero_flatten_bucket, zero_flatten_norm_bucket[_f32]) made in order:
checked bit for bit on random shards cut into random buckets, in all four
flatten modes, with and without the norm partials, with buckets of more than
64 segments (several launches each), and over back-to-back accumulating
calls on one destination, where each call's first launch must wait for the
previous call's unordered ones.  The per-bucket calls themselves are held to
the oracle elsewhere (test_gpu_parity, test_gpu_random)."""
import numpy as np
import pytest
import torch

import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _finite16(rng, k):
    b = rng.integers(0, 1 << 16, k, dtype=np.uint16)
    b[(b & 0x7C00) == 0x7C00] &= 0xBBFF            # no inf/NaN: every exact sum stays defined
    return b


def _case(seed, n, max_seg, misalign, bucket):
    rng = np.random.default_rng(seed)
    numels, segs = shardgen.random_segments(rng, n, max_seg, misalign)
    srcs = [H.to_dev16(_finite16(rng, k)) for k in numels]
    arr, k = Z.make_segments([(srcs[t].data_ptr(), so, do, c) for t, so, do, c in segs])
    buckets = [Z.zero_bucket_segments(arr, k, b, min(n, b + bucket)) for b in range(0, n, bucket)]
    return rng, srcs, buckets


def _per_bucket(buckets, dst, n, dtype, acc, partials):
    off = 0
    for segs, k in buckets:
        if partials is None:
            Z.zero_flatten_bucket(segs, k, dst, n, dtype, acc)
        elif dtype == Z.ZERO_F16:
            Z.zero_flatten_norm_bucket(segs, k, dst, partials, n, acc, off)
        else:
            Z.zero_flatten_norm_bucket_f32(segs, k, dst, partials, n, acc, off)
        off += Z.zero_flatten_norm_partials(segs, k)


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("dtype,acc", [(Z.ZERO_F16, False), (Z.ZERO_F16, True), (Z.ZERO_F32, False),
                                       (Z.ZERO_F32, True)])
@pytest.mark.parametrize("case", range(3))
def test_buckets_match_per_bucket_calls(case, dtype, acc, norm):
    n = [37_001, 400_003, 1_000_000][case]
    bucket = [4_096, 50_000, 131_072][case]
    rng, srcs, buckets = _case(1000 * case + 10 * dtype + acc, n, max(1, n // 9), case != 1, bucket)
    plan = Z.BucketPlan(buckets)
    H.log(f"buckets case {case}: n={n} buckets={len(plan)} segments={plan.nsegs} dtype={dtype} acc={acc} "
          f"norm={norm}")
    if dtype == Z.ZERO_F16:
        dst0 = H.to_dev16(_finite16(rng, n))
    else:
        dst0 = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    count = plan.partials()
    ref_p = new_p = None
    if norm:
        ref_p = torch.full((count * Z.NORM_PARTIAL_BYTES,), 0xA5, dtype=torch.uint8, device="cuda")
        new_p = torch.full_like(ref_p, 0x5A)
    ref, new = dst0.clone(), dst0.clone()
    _per_bucket(plan, ref, n, dtype, acc, ref_p)
    Z.zero_flatten_buckets(plan, new, n, dtype, acc, new_p)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.uint8), new.view(torch.uint8))
    if norm:
        assert torch.equal(ref_p, new_p)


@pytest.mark.parametrize("dtype", [Z.ZERO_F16, Z.ZERO_F32])
def test_back_to_back_accumulating_calls(dtype):
    """Five accumulating multi-bucket calls in a row on one destination, with
    norm partials on the last: every call's first launch must wait for the
    previous call's unordered launches, or a read-modify-write is lost."""
    n, bucket = 2_000_003, 65_536
    _, srcs, buckets = _case(77 + dtype, n, 40_000, True, bucket)
    plan = Z.BucketPlan(buckets)
    assert len(plan) == 31
    count = plan.partials()
    zero = torch.zeros(n, dtype=torch.float16 if dtype == Z.ZERO_F16 else torch.float32, device="cuda")
    ref, new = zero.clone(), zero.clone()
    ref_p = torch.zeros(count * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
    new_p = torch.ones_like(ref_p)
    for k in range(5):
        last = k == 4
        _per_bucket(plan, ref, n, dtype, True, ref_p if last else None)
        Z.zero_flatten_buckets(plan, new, n, dtype, True, new_p if last else None)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.uint8), new.view(torch.uint8))
    assert torch.equal(ref_p, new_p)


def test_buckets_of_many_segments():
    """Buckets of more than 64 segments take several launches each; all of
    them but the call's first are unordered."""
    n = 600_000
    _, srcs, buckets = _case(5, n, 700, False, 200_000)
    plan = Z.BucketPlan(buckets)
    assert len(plan) == 3 and all(k > 64 for _, k in plan)
    count = plan.partials()
    ref = torch.zeros(n, dtype=torch.float16, device="cuda")
    new = torch.ones_like(ref)
    ref_p = torch.zeros(count * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
    new_p = torch.ones_like(ref_p)
    _per_bucket(plan, ref, n, Z.ZERO_F16, False, ref_p)
    Z.zero_flatten_buckets(plan, new, n, Z.ZERO_F16, False, new_p)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.uint8), new.view(torch.uint8)) and torch.equal(ref_p, new_p)


@pytest.mark.parametrize("any_order", [False, True])
def test_bucketed_steps_against_oracle(any_order):
    """A bucketed shard stepped through the stepper both ways, each held to
    the oracle (fused step: flatten with partials, decide, Adam)."""
    w = shardgen.workload("tiny")
    w.bucket_elems = 777
    r = H.start(w, fused=True, any_order=any_order)
    for _ in range(4):
        H.step(r)
    assert len(r.dev.buckets) > 1 and r.stats["fp32_not_bitwise"] == 0, r.stats


def test_copy_right_after_the_call_sees_every_bucket():
    """The call's last launch keeps the dispatch barrier, so whatever waits on
    the stream's last packet -- here a copy to the host queued straight after
    the call, with no synchronisation in between -- sees every bucket's
    stores, including those of the unordered launches before it."""
    n, bucket = 3_000_017, 50_000
    rng, srcs, buckets = _case(91, n, 30_000, True, bucket)
    plan = Z.BucketPlan(buckets)
    assert len(plan) == 61
    ref = torch.zeros(n, dtype=torch.float16, device="cuda")
    _per_bucket(plan, ref, n, Z.ZERO_F16, False, None)
    ref_host = ref.view(torch.int16).cpu()
    for k in range(3):
        dst = torch.full((n,), float(k + 1), dtype=torch.float16, device="cuda")
        Z.zero_flatten_buckets(plan, dst, n, Z.ZERO_F16, False)
        assert torch.equal(dst.view(torch.int16).cpu(), ref_host), k
