"""The shard's state arena (stepper.state_arena), checked on the CPU: every
array starts 64 KiB x its index past a 2 MiB boundary, the arrays are
disjoint and in order, zero-filled, of the requested sizes and dtypes, and
they stay valid after the caller drops everything but the views."""
import gc

import pytest
import torch

from zero_partitioned_mixed_flatten_amd.stepper import ARENA_ALIGN, ARENA_STAGGER, state_arena


@pytest.mark.parametrize("n", [1, 7, 4099, (1 << 20) + 3, 3 << 20])
def test_arena_layout(n):
    specs = [("p32", n, torch.float32), ("m32", n, torch.float32), ("v32", n, torch.float32),
             ("grad16", n, torch.float16), ("p16", n, torch.float16), ("err", n + 5, torch.float32)]
    a = state_arena("cpu", specs)
    assert list(a) == [s[0] for s in specs]
    prev_end = None
    for k, (name, numel, dtype) in enumerate(specs):
        t = a[name]
        assert t.dtype == dtype and t.numel() == numel and t.is_contiguous()
        assert t.data_ptr() % ARENA_ALIGN == k * ARENA_STAGGER
        assert t.data_ptr() % 16 == 0
        assert torch.count_nonzero(t).item() == 0
        if prev_end is not None:
            assert t.data_ptr() >= prev_end            # disjoint, in the given order
        prev_end = t.data_ptr() + numel * t.element_size()


def test_arena_views_keep_it_alive():
    a = state_arena("cpu", [("x", 1000, torch.float32), ("y", 1000, torch.float16)])
    x, y = a["x"], a["y"]
    del a
    gc.collect()
    x.fill_(3.0)
    y.fill_(-1.0)
    assert float(x.sum()) == 3000.0 and float(y.float().sum()) == -1000.0
    assert x.data_ptr() + 4000 <= y.data_ptr()
