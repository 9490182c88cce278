"""GPU parity tests of the offloaded step (the ZeRO-Offload form): the device
flattens the per-layer fp16 gradients into its flat partition, the gradient
comes down to pinned host memory in chunks, the CPU takes the exact norm, the
decision and the AdamW update of the host-resident fp32 state, and the fp16
parameters go back up -- against the oracle on the same seeded inputs.

Contract: host state bitwise (including the exact sum), host p32, m32, v32
bitwise over the whole shard, device p16 bitwise, and the staged gradient
bitwise equal to the oracle's flatten."""
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


class Offload:
    def __init__(self, w, threads=0, chunk=1 << 20, device_decides=True):
        self.w = w
        n = w.n
        p32 = shardgen.master_params(w)
        self.dev = Z.OffloadStep(n, threads=threads, chunk_elems=chunk, device_decides=device_decides)
        if n:
            self.dev.p32.copy_(torch.from_numpy(p32))
            self.dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
        self.dev.init_state(w.scale0)
        self.st = O.new_state(w.scale0)
        self.hp_o = H.oracle_hparams(w.hp)
        self.hp_d = H.device_hparams(w.hp)
        self.p32, self.m32, self.v32 = p32.copy(), np.zeros_like(p32), np.zeros_like(p32)
        self.p16 = shardgen.to_f16_bits(p32)
        self.k = 0

    def step(self):
        self.k += 1
        w = self.w
        gpart = shardgen.grad_partition(w, self.k, self.st.loss_scale)
        srcs = shardgen.source_tensors(w.layout, gpart)
        del gpart
        dsrcs = [H.to_dev16(s) for s in srcs]
        H.log(f"offload {w.name} n={w.n} step {self.k} chunk={self.dev.chunk} threads={self.dev.ctx.threads} "
              f"device_decides={self.dev.device_decides}")
        self.dev.set_segments(dsrcs, w.layout.segments, w.bucket_elems)
        self.dev.step(self.hp_d)
        grad = np.empty(w.n, np.uint16)
        O.flatten(srcs, w.layout.segments, grad)
        s, o = O.norm_overflow(grad)
        O.decide(self.st, self.hp_o, s, o)
        O.adam_update(self.st, self.p16, self.p32, self.m32, self.v32, grad)
        torch.cuda.synchronize()
        H.log(f"offload {w.name} step {self.k}: done, overflow={o} norm={self.st.grad_norm:.6g}")
        H.compare_state(self.dev.read_state(), self.st, H.exact_units(grad) if (not o and w.n <= (1 << 27)) else None)
        assert np.array_equal(self.dev.host_grad16.numpy().view(np.uint16)[:w.n], grad)
        for a, b in ((self.dev.p32, self.p32), (self.dev.m32, self.m32), (self.dev.v32, self.v32)):
            assert a.numpy()[:w.n].tobytes() == b.tobytes()
        assert np.array_equal(H.bits16(self.dev.p16)[:w.n], self.p16)
        del dsrcs


@pytest.mark.parametrize("device_decides", [True, False])
@pytest.mark.parametrize("chunk", [256, 4096, 1 << 20])       # 256: 4096 chunks, the most allowed
def test_offload_tiny_full_parity(chunk, device_decides):
    r = Offload(shardgen.workload("tiny"), chunk=chunk, device_decides=device_decides)
    for _ in range(3):
        r.step()


@pytest.mark.parametrize("device_decides", [True, False])
@pytest.mark.parametrize("n", [1, 7, 65_536 * 3 + 5])
def test_offload_ragged(n, device_decides):
    r = Offload(_small(f"offload{n}", n, seed=300 + n), threads=3, chunk=64, device_decides=device_decides)
    for _ in range(2):
        r.step()


@pytest.mark.parametrize("device_decides", [True, False])
def test_offload_empty(device_decides):
    w = _small("offload-empty", 0, seed=0)
    w.layout = shardgen.ShardLayout("empty", 0, 1, 0, 0, 0, [], [], [])
    r = Offload(w, device_decides=device_decides)
    r.step()
    assert r.dev.read_state().step == 1


@pytest.mark.parametrize("device_decides", [True, False])
def test_offload_gpt2_shard_full_size(device_decides):
    r = Offload(shardgen.workload("gpt2"), chunk=1 << 23, device_decides=device_decides)
    for _ in range(2):
        r.step()


@pytest.mark.parametrize("device_decides", [True, False])
def test_offload_skip_leaves_everything(device_decides):
    w = _small("offload-skip", 100_000, seed=17)
    w.inject = {2: 0x7E00}
    r = Offload(w, chunk=8192, device_decides=device_decides)
    r.step()
    snap = [t.clone() for t in (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)]
    r.step()
    s = r.dev.read_state()
    assert s.skip == 1 and s.loss_scale == w.scale0 / 2
    for a, b in zip(snap, (r.dev.p16, r.dev.p32, r.dev.m32, r.dev.v32)):
        assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()
    r.step()
    assert r.dev.read_state().step == 2


def test_offload_matches_device_step():
    """The offloaded step and the all-device step take the same decision and
    produce the same parameters, bit for bit."""
    w = _small("offload-vs-device", 500_003, seed=23, max_seg=90_000)
    off = Offload(w, chunk=1 << 16, device_decides=False)       # the CPU decides here
    dev = H.start(w, fused=True)
    for _ in range(2):
        off.step()
        H.step(dev)
        assert bytes(off.dev.read_state()) == bytes(dev.dev.read_state())
        assert torch.equal(off.dev.p16.view(torch.int16), dev.dev.p16.view(torch.int16))
        assert off.dev.p32.numpy().tobytes() == dev.dev.p32.cpu().numpy().tobytes()
