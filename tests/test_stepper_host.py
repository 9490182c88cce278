"""The shard's state arena (stepper.StateArena), checked on the CPU: every
array starts 64 KiB x its index past a 2 MiB boundary, the arrays are
disjoint and in order, zero-filled, of the requested sizes and dtypes, they
stay valid after the caller drops the arena object, and every byte around
them holds the canary that intact() checks."""
import gc

import pytest
import torch

from zero_partitioned_mixed_flatten_amd.stepper import ARENA_ALIGN, ARENA_CANARY, ARENA_STAGGER, StateArena


def _specs(n):
    return [("p32", n, torch.float32), ("m32", n, torch.float32), ("v32", n, torch.float32),
            ("grad16", n, torch.float16), ("p16", n, torch.float16), ("bits", (n + 7) // 8, torch.uint8)]


@pytest.mark.parametrize("n", [1, 7, 4099, (1 << 20) + 3, 3 << 20])
def test_arena_layout(n):
    specs = _specs(n)
    arena = StateArena("cpu", specs)
    a = arena.arrays
    assert list(a) == [s[0] for s in specs]
    base = arena.tensor.data_ptr()
    prev_end = base + ARENA_ALIGN                     # at least 2 MiB of guard before the first array
    for k, (name, numel, dtype) in enumerate(specs):
        t = a[name]
        assert t.dtype == dtype and t.numel() == numel and t.is_contiguous()
        assert t.data_ptr() % ARENA_ALIGN == k * ARENA_STAGGER
        assert t.data_ptr() >= prev_end + (ARENA_STAGGER if k else 0)   # disjoint, in order, gapped
        assert torch.count_nonzero(t).item() == 0
        prev_end = t.data_ptr() + numel * t.element_size()
    assert prev_end + ARENA_ALIGN <= base + arena.tensor.numel()         # and after the last one
    covered = sum(hi - lo for lo, hi in arena.gaps) + sum(t.numel() * t.element_size() for t in a.values())
    assert covered == arena.tensor.numel()                             # gaps + arrays tile the arena
    assert all(bool((arena.tensor[lo:hi] == ARENA_CANARY).all()) for lo, hi in arena.gaps)
    assert arena.intact()


def test_arena_views_keep_it_alive():
    arena = StateArena("cpu", [("x", 1000, torch.float32), ("y", 1000, torch.float16)])
    x, y = arena.arrays["x"], arena.arrays["y"]
    del arena
    gc.collect()
    x.fill_(3.0)
    y.fill_(-1.0)
    assert float(x.sum()) == 3000.0 and float(y.float().sum()) == -1000.0
    assert x.data_ptr() + 4000 <= y.data_ptr()


@pytest.mark.parametrize("where", ["before_first", "after_first", "before_last", "after_last"])
def test_intact_sees_a_store_just_outside_an_array(where):
    """Writes inside the arrays leave the guard intact; one byte stored just
    outside any array (here from the host, standing in for a kernel that
    overruns) is caught."""
    arena = StateArena("cpu", _specs(4099))
    for t in arena.arrays.values():
        t.view(torch.uint8).fill_(0xFF)               # every byte of every array, and nothing else
    assert arena.intact()
    first, last = arena.arrays["p32"], arena.arrays["bits"]
    off = {"before_first": first.data_ptr() - 1,
           "after_first": first.data_ptr() + first.numel() * 4,
           "before_last": last.data_ptr() - 1,
           "after_last": last.data_ptr() + last.numel()}[where] - arena.tensor.data_ptr()
    arena.tensor[off] = 0
    assert not arena.intact()


def test_step_arrays_cannot_be_rebound():
    """The step's calls pass the addresses taken when it was made, so its
    arrays (and those of the 1-bit form) are written in place; rebinding one
    is an error instead of being silently ignored.  Host only: nothing is
    launched."""
    import zero_partitioned_mixed_flatten_amd as Z
    for step in (Z.ShardStep(1000, device="cpu"), Z.OneBitStep(1000, warmup=2, device="cpu")):
        names = ["p32", "m32", "v32", "grad16", "p16", "state"]
        if isinstance(step, Z.OneBitStep):
            names += ["err_w", "err_s", "bits_w", "bits_s"]
        for name in names:
            old = getattr(step, name)
            with pytest.raises(AttributeError, match="in place"):
                setattr(step, name, torch.zeros_like(old))
            assert getattr(step, name) is old
        step.p32.fill_(1.5)                       # in place is the way
        assert float(step.arena.arrays["p32"][0]) == 1.5
        step.fused = True                         # ordinary attributes stay assignable
