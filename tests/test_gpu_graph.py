"""The fused step under HIP graph capture: flatten with exact-norm partials,
decide and the update captured once in a graph and replayed, with eager work
(new gradient values copied into the captured source tensors, reads of the
state) and synchronisations between the replays; every replay must equal the
same step run eagerly on a twin set of buffers, bit for bit.  The step issues
no memset and its arrival counters re-arm themselves, so nothing in it
depends on being launched eagerly.  For 1-bit Adam the one captured step
replays across the hand-over from the warm-up to the compression stage (the
device picks the stage)."""
import numpy as np
import pytest
import torch

import shardgen

pytestmark = pytest.mark.gpu

import gpu_harness as H  # noqa: E402
import zero_partitioned_mixed_flatten_amd as Z  # noqa: E402


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.float16 else t.view(torch.int32)


@pytest.mark.parametrize("onebit,bucket", [(False, 0), (True, 0), (False, 100_000)])
def test_fused_step_graph_replays_match_eager(onebit, bucket):
    """bucket > 0: the partition is flattened in buckets, which the eager twin
    issues without dispatch barriers between them and the capture records as
    ordinary graph nodes."""
    rng = np.random.default_rng(61)
    n = 600_011
    numels, segs = shardgen.random_segments(rng, n, 90_000)
    w = shardgen.workload("tiny")
    w.layout = shardgen.ShardLayout("graph", n, 1, 0, 0, n, [f"t{i}" for i in range(len(numels))], numels, segs)
    p32 = shardgen.master_params(w)
    hp = H.device_hparams(w.hp)

    def make():
        d = Z.OneBitStep(n, warmup=2) if onebit else Z.ShardStep(n, fused=True)
        d.p32.copy_(torch.from_numpy(p32))
        d.p16.copy_(d.p32.half())
        d.init_state(w.scale0)
        return d

    eager, graphed = make(), make()
    src_e = [torch.zeros(k, dtype=torch.float16, device="cuda") for k in numels]
    src_g = [torch.zeros(k, dtype=torch.float16, device="cuda") for k in numels]
    eager.set_segments(src_e, segs, bucket)
    graphed.set_segments(src_g, segs, bucket)
    assert len(eager.buckets) == (7 if bucket else 1)

    def load(k):
        gpart = shardgen.grad_partition(w, k, 2.0 ** 16)
        for dst in (src_e, src_g):
            for t, a in zip(dst, shardgen.source_tensors(w.layout, gpart)):
                t.copy_(torch.from_numpy(a.view(np.float16)))

    def body(d):
        d.flatten_norm()
        d.decide(hp)
        if onebit:
            d.update()                                  # warm-up or compression: the device decides
        else:
            d.adam()

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            body(graphed)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capturing ran nothing: both twins are still at step 0
    assert graphed.read_state().step == 0
    for k in range(1, 7):
        load(k)                                         # eager work between replays
        torch.cuda.synchronize()
        H.log(f"graph replay {k} onebit={onebit}")
        g.replay()
        body(eager)
        torch.cuda.synchronize()
        a, b = eager.read_state(), graphed.read_state()
        assert bytes(a) == bytes(b), (a.as_dict(), b.as_dict())
        names = ["grad16", "p16", "p32", "m32", "v32"] + (["err_w", "err_s", "bits_w", "bits_s", "onebit"]
                                                          if onebit else [])
        for name in names:
            x, y = getattr(eager, name), getattr(graphed, name)
            if x.dtype in (torch.float16, torch.float32):
                x, y = _bits(x), _bits(y)
            assert torch.equal(x, y), (k, name)
        if onebit:                                      # the compression stage has started after step 2
            assert (graphed.read_onebit().scale_w != 0.0) == (k > 2), k
    assert eager.read_state().step == 6
