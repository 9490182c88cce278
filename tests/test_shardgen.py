"""Checks of the seeded input generator: layouts have the sizes the model
shapes imply and draws are reproducible and thread-count independent."""
import numpy as np

import shardgen


def test_gpt2_layout():
    L = shardgen.gpt2_layout()
    assert L.psi == 1_557_611_200 == 48 * 30_740_800 + 50257 * 1600 + 1024 * 1600 + 3200
    assert L.n == L.psi // 16 == 97_350_700
    assert len(L.segments) == 39
    assert L.segments[0][1] > 0                       # the shard starts inside a tensor
    _check_cover(L)


def test_100b_layout():
    L = shardgen.gpt100b_layout()
    assert L.n == 125 * 50_384_384 // 25 == 251_921_920
    assert len(L.segments) == 60
    _check_cover(L)


def test_1t_layout():
    L = shardgen.gpt1t_layout()
    assert L.n == 976_562_500 and len(L.segments) == 17
    assert L.n % 8 == 4                               # a ragged vector tail
    _check_cover(L)


def _check_cover(L):
    d = 0
    for t, so, do, cnt in L.segments:
        assert do == d and cnt > 0 and so + cnt <= L.tensor_numels[t]
        d += cnt
    assert d == L.n


def test_draws_reproducible_and_chunk_stable():
    a = shardgen.standard_normal_f32(3 * shardgen.CHUNK + 5, [0, 9])
    b = shardgen.standard_normal_f32(3 * shardgen.CHUNK + 5, [0, 9])
    assert np.array_equal(a, b)
    head = shardgen.standard_normal_f32(shardgen.CHUNK + 1, [0, 9])
    assert np.array_equal(a[:shardgen.CHUNK + 1], head)
    assert abs(float(a.std()) - 1.0) < 1e-3


def test_injection_and_sentinel():
    w = shardgen.workload("stress")
    w.layout = shardgen.single_tensor_layout(1 << 16)
    g = shardgen.grad_partition(w, 3, w.scale0)
    pos = shardgen.injection_position(w, 3)
    assert g[pos] == 0x7C00
    assert int(np.sum((g & 0x7C00) == 0x7C00)) == 1
    L = shardgen.gpt2_layout()
    small = shardgen.ShardLayout("x", 0, 1, 0, 0, 4, ["a"], [10], [(0, 3, 0, 4)])
    t = shardgen.source_tensors(small, np.arange(4, dtype=np.uint16))
    assert list(t[0]) == [0x7E00] * 3 + [0, 1, 2, 3] + [0x7E00] * 3
    assert L.n > 0


def test_stress_injections_are_the_only_non_finite_values_full_shard():
    """On the full 97M-element stress shard at S = 2^24 (sigma 1e-4: 65520 is 39
    sigma away), the injected +inf (step 3) and NaN (step 7) are the only
    non-finite fp16 values, and a clean step has none."""
    w = shardgen.workload("stress")
    for step, bits in ((3, 0x7C00), (7, 0x7E00), (4, None)):
        g = shardgen.grad_partition(w, step, w.scale0)
        bad = np.flatnonzero((g & 0x7C00) == 0x7C00)
        if bits is None:
            assert bad.size == 0
        else:
            assert bad.tolist() == [shardgen.injection_position(w, step)] and g[bad[0]] == bits
