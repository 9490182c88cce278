"""Seeded random sweep of the GPU step against the oracle: each case draws a
shard size (tiny to several workgroups with a ragged tail), a segment layout
(aligned or not, one to hundreds of segments, bucketed or not), the
hyperparameters, the gradient magnitude and loss scale (so clipping, growth
and overflow all occur), and optionally an inf or NaN in one step.  Every
step is held to the full contract (bitwise state, partition, p16, and p32/m32/v32
counted bitwise) for the fused and separate fp16 paths, the fp32
accumulation path and the 1-bit Adam compression stage; and random fp32
partitions off the fast path through the exact wide pass."""
import numpy as np
import pytest

import oracle as O
import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _draw(case: int, tag: str) -> shardgen.Workload:
    rng = np.random.default_rng([case, sum(map(ord, tag))])
    n = int(rng.choice([rng.integers(1, 70), rng.integers(70, 9000), rng.integers(9000, 300_000)]))
    misalign = bool(rng.integers(0, 2))
    max_seg = int(rng.choice([1 + n // 200, 1 + n // 7, n]))
    numels, segs = shardgen.random_segments(rng, n, max(1, max_seg), misalign)
    w = shardgen.workload("tiny")
    w.name = f"{tag}{case}"
    w.layout = shardgen.ShardLayout(w.name, n, 1, 0, 0, n, [f"t{i}" for i in range(len(numels))], numels, segs)
    w.seed = int(rng.integers(0, 2 ** 31))
    w.sigma_p = float(rng.choice([0.02, 1.0]))
    w.sigma_g = float(rng.choice([1e-6, 1e-3, 1e-1]))
    w.scale0 = float(2.0 ** int(rng.integers(0, 25)))
    w.bucket_elems = int(rng.choice([0, 0, 1 + n // 3]))
    w.hp = shardgen.HParams(lr=float(rng.choice([0.0, 1e-4, 3e-3])), beta1=float(rng.choice([0.0, 0.9, 0.99])),
                            beta2=float(rng.choice([0.0, 0.95, 0.999])), eps=float(rng.choice([1e-8, 1e-6])),
                            weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
                            max_grad_norm=float(rng.choice([0.0, 1e-3, 1.0, 1e3])),
                            backoff=float(rng.choice([0.5, 0.25])), growth=float(rng.choice([2.0, 4.0])),
                            min_scale=1.0, growth_interval=int(rng.choice([1, 2, 20])))
    if rng.integers(0, 3) == 0:
        w.inject = {int(rng.integers(1, 4)): int(rng.choice([0x7C00, 0xFC00, 0x7E00, 0xFFFF]))}
    return w


@pytest.mark.parametrize("case", range(64))
def test_random_fp16_step(case):
    w = _draw(case, "f16-")
    r = H.start(w, fused=bool(case % 2))
    for _ in range(3):
        H.step(r)
    assert r.stats["fp32_not_bitwise"] == 0, r.stats


@pytest.mark.parametrize("case", range(32))
def test_random_accumulation_step(case):
    w = _draw(case, "f32-")
    r = H.start_accum(w, int(1 + case % 3), fused=bool(case % 2))
    for _ in range(2):
        H.step_accum(r)


@pytest.mark.parametrize("case", range(32))
def test_random_onebit_steps(case):
    from test_gpu_onebit import OneBitRun
    w = _draw(case, "1b-")
    w.bucket_elems = 0
    r = OneBitRun(w, warmup=int(case % 3))
    for _ in range(4):
        r.step()


@pytest.mark.parametrize("case", range(32))
def test_random_fp32_partition_exact_norm(case):
    """Random fp32 partitions off the fast path (any binary32 magnitude, off
    the 2^-24 grid, with zeros, subnormals and sometimes an inf or NaN): the
    standalone fp32 reduction, and the fused fp32 flatten folded by
    zero_shard_decide_f32, each take the oracle's decision from its plain exact
    sum, bit for bit."""
    import torch
    rng = np.random.default_rng([case, 9191])
    n = int(rng.choice([rng.integers(1, 70), rng.integers(70, 9000), rng.integers(9000, 400_000)]))
    lo = int(rng.integers(-149, 100))
    hi = int(rng.integers(lo + 1, 129))
    mant = rng.integers(1 << 23, 1 << 24, n).astype(np.float64)
    base = np.minimum(mant * np.exp2(rng.integers(lo, hi, n) - 23.0), float(np.finfo(np.float32).max))
    base = (base * np.where(rng.integers(0, 2, n) == 1, -1, 1)).astype(np.float32)
    base[rng.integers(0, n, n // 5)] = 0.0
    if rng.integers(0, 4) == 0:
        base[int(rng.integers(0, n))] = rng.choice([np.inf, -np.inf, np.nan])
    scale0 = float(2.0 ** int(rng.integers(0, 25)))
    clip = float(rng.choice([0.0, 1.0]))
    hp_d, hp_o = Z.hparams(max_grad_norm=clip), O.hparams(max_grad_norm=clip)
    ref = O.new_state(scale0)
    O.decide(ref, hp_o, *O.norm_overflow_f32(base))
    # standalone
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(16, Z.zero_norm_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st, scale0)
    H.log(f"random fp32 norm case {case}: n={n} exponents [{lo}, {hi})")
    Z.zero_shard_norm_overflow_f32(torch.from_numpy(base).cuda(), n, hp_d, st, ws)
    s = Z.read_state(st)
    assert s.wide_pending == 0
    H.compare_state(s, ref, None)
    # fused: the partition is what an fp32 widen of zero source values leaves plus the crafted values
    numels, segs = shardgen.random_segments(rng, n, max(1, n // 3), True)
    srcs = [np.zeros(k, np.uint16) for k in numels]
    dsrcs = [H.to_dev16(x) for x in srcs]
    arr, k = Z.make_segments([(dsrcs[t].data_ptr(), so, do, c) for t, so, do, c in segs])
    count = Z.zero_flatten_norm_partials(arr, k)
    partials = torch.empty(max(1, count) * Z.NORM_PARTIAL_BYTES, dtype=torch.uint8, device="cuda")
    dws = torch.empty(max(16, Z.zero_decide_workspace_bytes(count)), dtype=torch.uint8, device="cuda")
    dst = torch.from_numpy(base.copy()).cuda()
    Z.zero_flatten_norm_bucket_f32(arr, k, dst, partials, n, True)         # dst + 0 leaves every value
    Z.zero_step_state_init(st, scale0)
    Z.zero_shard_decide_f32(partials, count, dst, n, hp_d, st, dws)
    s2 = Z.read_state(st)
    assert bytes(s2) == bytes(s) or (s2.overflow == s.overflow == 1), (s2.as_dict(), s.as_dict())
