"""Pins for the oracle's flatten against numpy: a bit copy must equal the
concatenation of the source slices; the accumulating forms must equal numpy's
float16 / float32 additions (independent library routines)."""
import numpy as np
import pytest

import shardgen


def _random_case(seed, n=5000, max_seg=700):
    rng = np.random.default_rng(seed)
    numels, segs = shardgen.random_segments(rng, n, max_seg)
    srcs = [rng.integers(0, 0x7C00, k).astype(np.uint16) | (rng.integers(0, 2, k).astype(np.uint16) << 15)
            for k in numels]
    return rng, srcs, segs


@pytest.mark.parametrize("seed", range(4))
def test_copy_is_concatenation(oracle, seed):
    rng, srcs, segs = _random_case(seed)
    n = sum(c for *_, c in segs)
    dst = np.full(n, 0xABCD, np.uint16)
    oracle.flatten(srcs, segs, dst)
    ref = np.concatenate([srcs[t][so:so + c] for t, so, _, c in segs])
    assert np.array_equal(dst, ref)


def test_uncovered_elements_untouched(oracle):
    rng, srcs, segs = _random_case(11)
    holes = [s for i, s in enumerate(segs) if i % 3 != 1]
    n = sum(c for *_, c in segs)
    dst = np.full(n, 0x1234, np.uint16)
    oracle.flatten(srcs, holes, dst)
    mask = np.zeros(n, bool)
    for _, _, do, c in holes:
        mask[do:do + c] = True
    assert np.all(dst[~mask] == 0x1234)


@pytest.mark.parametrize("seed", range(3))
def test_accumulate_f16_is_numpy_half_add(oracle, seed):
    rng, srcs, segs = _random_case(20 + seed)
    n = sum(c for *_, c in segs)
    dst0 = (rng.standard_normal(n).astype(np.float32) * 300).astype(np.float16).view(np.uint16)
    srcs = [(rng.standard_normal(s.size).astype(np.float32) * 300).astype(np.float16).view(np.uint16)
            for s in srcs]
    dst = dst0.copy()
    oracle.flatten(srcs, segs, dst, accumulate=True)
    cat = np.concatenate([srcs[t][so:so + c] for t, so, _, c in segs])
    with np.errstate(over="ignore"):
        ref = (dst0.view(np.float16) + cat.view(np.float16)).view(np.uint16)
    assert np.array_equal(dst, ref)


def test_accumulate_f16_overflow_and_subnormal(oracle):
    a = np.array([0x7BFF, 0x0001, 0x8001, 0x3C00, 0x0200], np.uint16)
    b = np.array([0x7BFF, 0x0001, 0x0001, 0x1000, 0x0200], np.uint16)
    dst = a.copy()
    oracle.flatten([b], [(0, 0, 0, b.size)], dst, accumulate=True)
    with np.errstate(over="ignore"):
        ref = (a.view(np.float16) + b.view(np.float16)).view(np.uint16)
    assert np.array_equal(dst, ref) and dst[0] == 0x7C00


@pytest.mark.parametrize("accumulate", [False, True])
def test_f32_destination(oracle, accumulate):
    rng, srcs, segs = _random_case(30)
    n = sum(c for *_, c in segs)
    dst0 = rng.standard_normal(n).astype(np.float32)
    dst = dst0.copy()
    oracle.flatten(srcs, segs, dst, accumulate=accumulate)
    cat = np.concatenate([srcs[t][so:so + c] for t, so, _, c in segs]).view(np.float16).astype(np.float32)
    ref = dst0 + cat if accumulate else cat
    assert np.array_equal(dst.view(np.uint32), ref.view(np.uint32))
