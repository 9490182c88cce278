"""The fp16 reduction that allocates nothing (zero_shard_norm_overflow_noalloc)
against the entry point it varies (zero_shard_norm_overflow with a caller
workspace), through the C ABI: the whole 128-byte step state bit for bit,
on calls in a row whose sizes shrink, so that the second call reads the
library's scratch array right after a larger call has left its partials
there; and the decision against the oracle."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _grad(n, seed, inject=None):
    rng = np.random.default_rng(seed)
    g = shardgen.to_f16_bits((rng.standard_normal(n) * 1e-3 * 2.0 ** 16).astype(np.float32))
    if inject is not None:
        g[inject[0]] = inject[1]
    return g


def _state_bytes(dev_state):
    torch.cuda.synchronize()
    return bytes(dev_state.cpu().numpy().tobytes())


def test_noalloc_matches_workspace_form_on_shrinking_calls():
    hp = Z.hparams()
    hp_o = O.hparams()
    st_ws = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    st_na = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st_ws, 2.0 ** 16)
    Z.zero_step_state_init(st_na, 2.0 ** 16)
    ref = O.new_state(2.0 ** 16)
    # 256 workgroups, then 193 (an inf in the middle), then 2, then one
    cases = [((1 << 26) + 5, 1, None), (3 * (1 << 20) + 7, 2, (1_234_567, 0x7C00)), (20_000, 3, None),
             (1000, 4, None)]
    for n, seed, inject in cases:
        g = _grad(n, seed, inject)
        dg = H.to_dev16(g)
        ws = torch.empty(max(16, Z.zero_norm_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
        H.log(f"noalloc: n={n} seed={seed} inject={inject}")
        Z.zero_shard_norm_overflow(dg, n, hp, st_ws, ws)
        Z.zero_shard_norm_overflow_noalloc(dg, n, hp, st_na)
        a, b = _state_bytes(st_ws), _state_bytes(st_na)
        assert a == b, f"n={n}: step states differ"
        O.decide(ref, hp_o, *O.norm_overflow(g))
        H.compare_state(Z.read_state(st_na), ref, None if inject else H.exact_units(g))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # checked on the host before any device work: no launch happens
    hp = Z.hparams()
    st = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    g = torch.zeros(16, dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = Z.lib().zero_shard_norm_overflow_noalloc(g.data_ptr(), (1 << 30) + 1, C.byref(hp), st.data_ptr(), stream)
    assert rc == -3                          # ZERO_ERANGE
    rc = Z.lib().zero_shard_norm_overflow_noalloc(g.data_ptr(), 16, None, st.data_ptr(), stream)
    assert rc == -1                          # ZERO_EINVAL


def test_noalloc_at_its_largest_size():
    """n = 2^30, the largest size the scratch array takes: 256 workgroups of
    1024 threads, each thread summing its full 4096 values.  The partition is
    0.5 everywhere but at planted positions (the ends, the last vector, and
    random ones), so the exact sum is a closed form; both entry points give
    the same state bytes, the 128-bit sum is the closed form, and the
    decision is the oracle's."""
    from fractions import Fraction
    n = 1 << 30
    rng = np.random.default_rng(71)
    pos = np.unique(np.concatenate([np.array([0, 1, 7, 8, n - 9, n - 8, n - 1]), rng.integers(0, n, 64)]))
    bits = rng.integers(0, 0x7C00, pos.size, dtype=np.uint16) | (rng.integers(0, 2, pos.size, dtype=np.uint16) << 15)
    dg = torch.full((n,), 0.5, dtype=torch.float16, device="cuda")
    dg[torch.from_numpy(pos).cuda()] = H.to_dev16(bits)

    def units(b):                                   # x^2 in units of 2^-48 from the binary16 fields
        f, m = (int(b) >> 10) & 31, int(b) & 1023
        e = f - 25 if f else -24
        return (m | (1024 if f else 0)) ** 2 << (2 * e + 48)
    exact = (n - pos.size) * (1 << 46) + sum(units(b) for b in bits)
    hp = Z.hparams()
    st_ws = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    st_na = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st_ws, 2.0 ** 16)
    Z.zero_step_state_init(st_na, 2.0 ** 16)
    ws = torch.empty(Z.zero_norm_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    H.log(f"noalloc: n={n} (the largest size), closed-form sum")
    Z.zero_shard_norm_overflow(dg, n, hp, st_ws, ws)
    Z.zero_shard_norm_overflow_noalloc(dg, n, hp, st_na)
    assert _state_bytes(st_ws) == _state_bytes(st_na)
    ref = O.new_state(2.0 ** 16)
    O.decide(ref, O.hparams(), float(Fraction(exact, 1 << 48)), 0)
    H.compare_state(Z.read_state(st_na), ref, exact)
    del dg, ws
    torch.cuda.empty_cache()


def test_noalloc_under_graph_capture():
    """Code under HIP graph capture is one of the callers this entry point is
    for: the call is captured once (after one eager call, which looks up the
    scratch array's address) and replayed four times, with new gradient
    values copied in eagerly between the replays (an inf in one of them);
    after each replay the state equals, byte for byte, that of the workspace
    form run eagerly on a twin state."""
    n = 3 * (1 << 20) + 7
    hp = Z.hparams()
    st_g = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    st_e = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device="cuda")
    dg = torch.zeros(n, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(16, Z.zero_norm_workspace_bytes(n)), dtype=torch.uint8, device="cuda")
    Z.zero_step_state_init(st_g, 2.0 ** 16)
    Z.zero_shard_norm_overflow_noalloc(dg, n, hp, st_g)          # eager: the one-time address lookup
    Z.zero_step_state_init(st_g, 2.0 ** 16)
    Z.zero_step_state_init(st_e, 2.0 ** 16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            Z.zero_shard_norm_overflow_noalloc(dg, n, hp, st_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert Z.read_state(st_g).step == 0                          # capturing ran nothing
    for k in range(4):
        g16 = _grad(n, 200 + k, (777_777, 0x7C00) if k == 2 else None)
        dg.copy_(H.to_dev16(g16))
        torch.cuda.synchronize()
        H.log(f"noalloc graph replay {k + 1}")
        g.replay()
        Z.zero_shard_norm_overflow(dg, n, hp, st_e, ws)
        a, b = _state_bytes(st_e), _state_bytes(st_g)
        assert a == b, f"replay {k + 1}: states differ"
    assert Z.read_state(st_g).skipped_total == 1
