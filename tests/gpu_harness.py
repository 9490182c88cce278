"""Parity harness for the GPU tests: runs the HIP path and the oracle on the
same seeded inputs, step by step, and compares.

Full mode keeps the oracle's whole state.  Sampled mode (full-size shards)
keeps the oracle's state only at a fixed set of indices: the update is
elementwise, so the oracle computes those elements exactly as it would in a
full run, while the decision that drives them (exact norm, overflow, loss
scale, clip factor, bias corrections) still comes from the oracle's own pass
over the whole flattened gradient.

Contract checked every step:
  * flattened gradient: bitwise equal to the oracle's flatten;
  * step state: overflow, skip, loss scale, counters, exact sum (as a
    128-bit integer), sumsq, grad_norm and every fp32 factor bitwise;
  * fp16 parameters: bitwise; fp32 p, m, v: max relative error <= 1e-6
    (the count of elements that are not bitwise equal is reported; 0 is
    expected since both sides perform the same IEEE operations in the same
    order);
  * over the whole shard, p16 == fp16(p32) (torch's own cast).
"""
from __future__ import annotations

import math
import time
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import oracle as O
import shardgen
from floatcmp import same_floats32
import zero_partitioned_mixed_flatten_amd as Z

FP32_REL_TOL = 1e-6
TINY = float(np.finfo(np.float32).tiny)


def log(msg: str) -> None:
    print(f"[gpu-parity] {msg}", flush=True)


def to_dev16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.float16)).cuda()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return float(np.max(d / np.maximum(np.abs(ref.astype(np.float64)), TINY)))


def oracle_hparams(hp: shardgen.HParams) -> O.OracleHParams:
    return O.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_grad_norm, hp.backoff,
                     hp.growth, hp.min_scale, hp.growth_interval)


def device_hparams(hp: shardgen.HParams) -> Z.HParams:
    return Z.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.max_grad_norm, hp.backoff,
                     hp.growth, hp.min_scale, hp.growth_interval)


STATE_FIELDS = ("loss_scale", "beta1_pow", "beta2_pow", "step", "good_steps", "skipped_total", "overflow",
                "skip")
STEP_FIELDS = ("sumsq", "grad_norm", "gmul", "bc1", "bc2", "lr", "beta1", "beta2", "omb1", "omb2", "eps", "wd")


def compare_state(dev: Z.StepState, ref: O.OracleState, exact_units: Optional[int]) -> None:
    for f in STATE_FIELDS:
        assert getattr(dev, f) == getattr(ref, f), (f, getattr(dev, f), getattr(ref, f))
    fields = STEP_FIELDS if not ref.skip else ("sumsq", "grad_norm")
    for f in fields:
        a, b = getattr(dev, f), getattr(ref, f)
        if isinstance(a, float) and math.isnan(a):
            assert math.isnan(b), f
        else:
            assert np.float64(a).tobytes() == np.float64(b).tobytes(), (f, a, b)
    if exact_units is not None and not ref.skip:
        assert dev.as_dict()["sumsq_units"] == exact_units


def exact_units(grad: np.ndarray) -> int:
    """sum of squares of finite binary16 values in units of 2^-48, as a Python
    integer: each square * 2^48 is an integer below 2^80, split exactly into
    40-bit halves that numpy can add in int64 chunk by chunk."""
    total = 0
    for lo in range(0, grad.size, 1 << 22):
        x = grad[lo:lo + (1 << 22)].view(np.float16).astype(np.float64)
        v = x * x * 2.0 ** 48
        hi = np.floor(v / 2.0 ** 40)
        total += (int(hi.astype(np.int64).sum()) << 40) + int((v - hi * 2.0 ** 40).astype(np.int64).sum())
    return total


@dataclass
class Run:
    w: shardgen.Workload
    sample: Optional[np.ndarray] = None          # None: full oracle state
    dev: Z.ShardStep = None
    st: O.OracleState = None
    hp_o: O.OracleHParams = None
    hp_d: Z.HParams = None
    p16: np.ndarray = None
    p32: np.ndarray = None
    m32: np.ndarray = None
    v32: np.ndarray = None
    k: int = 0
    stats: dict = field(default_factory=lambda: {"fp32_not_bitwise": 0, "fp32_max_rel": 0.0})

    @property
    def n(self) -> int:
        return self.w.n

    def idx(self) -> np.ndarray:
        return np.arange(self.n) if self.sample is None else self.sample


def start(w: shardgen.Workload, sample: Optional[int] = None, seed: int = 77, fused: bool = False,
          any_order: bool = True) -> Run:
    """fused: run the step as flatten-with-norm-partials + decide + Adam;
    any_order: all buckets in one zero_flatten_buckets call (else one ordered
    call per bucket)."""
    r = Run(w)
    n = w.n
    if sample is not None and sample < n:
        rng = np.random.default_rng(seed)
        edges = []
        for _, _, do, c in w.layout.segments:          # both ends of every segment
            edges += [do, do + 1, do + c - 1, do + c - 2]
        edges += list(range(min(n, 64))) + list(range(max(0, n - 64), n))
        r.sample = np.unique(np.clip(np.concatenate([rng.integers(0, n, sample), np.array(edges)]), 0, n - 1))
    p32 = shardgen.master_params(w)
    r.dev = Z.ShardStep(n, fused=fused, any_order=any_order)
    if n:
        r.dev.p32.copy_(torch.from_numpy(p32))
        r.dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
    r.dev.init_state(w.scale0)
    i = r.idx()
    r.p32 = np.ascontiguousarray(p32[i])
    r.p16 = shardgen.to_f16_bits(r.p32)
    r.m32 = np.zeros_like(r.p32)
    r.v32 = np.zeros_like(r.p32)
    r.st = O.new_state(w.scale0)
    r.hp_o = oracle_hparams(w.hp)
    r.hp_d = device_hparams(w.hp)
    return r


def step(r: Run, check: bool = True, check_full_cast: bool = True, exact: bool = True) -> dict:
    """One step on both sides; returns a few timings/values for the log."""
    pending = prepare(r)
    enqueue(r, pending)
    return finish(r, pending, check, check_full_cast, exact)


def prepare(r: Run) -> tuple:
    """The next step's gradient sources, drawn on the host and uploaded
    (synchronously) to the device."""
    r.k += 1
    t0 = time.time()
    gpart = shardgen.grad_partition(r.w, r.k, r.st.loss_scale)
    srcs = shardgen.source_tensors(r.w.layout, gpart)
    del gpart
    dsrcs = [to_dev16(s) for s in srcs]
    return srcs, dsrcs, t0, time.time()


def enqueue(r: Run, pending: tuple, stream: Optional[torch.cuda.Stream] = None) -> None:
    """The device step on `stream` (torch's current stream if None); returns
    without waiting."""
    w, dsrcs = r.w, pending[1]
    log(f"{w.name} n={w.n} step {r.k}: launch (segments={len(w.layout.segments)}, bucket={w.bucket_elems}, "
        f"fused={r.dev.fused})")
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        r.dev.set_segments(dsrcs, w.layout.segments, w.bucket_elems)
        r.dev.step(r.hp_d)


def finish(r: Run, pending: tuple, check: bool = True, check_full_cast: bool = True, exact: bool = True) -> dict:
    """The oracle's side of the step, a device-wide synchronisation, and the
    comparison."""
    srcs, dsrcs, t0, t1 = pending
    k, w = r.k, r.w
    # oracle: its own flatten of the same sources, then the exact reduction and decision
    grad = np.empty(w.n, np.uint16)
    O.flatten(srcs, w.layout.segments, grad)
    sumsq, ovf = O.norm_overflow(grad)
    O.decide(r.st, r.hp_o, sumsq, ovf)
    i = r.idx()
    O.adam_update(r.st, r.p16, r.p32, r.m32, r.v32, np.ascontiguousarray(grad[i]))
    torch.cuda.synchronize()
    t2 = time.time()
    log(f"{w.name} step {k}: gpu done, overflow={ovf} norm={r.st.grad_norm:.6g} scale={r.st.loss_scale:g}")
    if not check:
        return {}
    dstate = r.dev.read_state()
    exact = exact_units(grad) if (exact and not ovf and w.n <= (1 << 27)) else None
    compare_state(dstate, r.st, exact)
    assert np.array_equal(bits16(r.dev.grad16)[:w.n], grad), "flattened gradient differs"
    it = torch.from_numpy(i).cuda()
    d16 = bits16(r.dev.p16[it])
    assert np.array_equal(d16, r.p16), f"p16 differs at {int(np.sum(d16 != r.p16))} elements"
    for name, dt, ref in (("p32", r.dev.p32, r.p32), ("m32", r.dev.m32, r.m32), ("v32", r.dev.v32, r.v32)):
        got = dt[it].cpu().numpy()
        e = rel_err(got, ref)
        r.stats["fp32_max_rel"] = max(r.stats["fp32_max_rel"], e)
        r.stats["fp32_not_bitwise"] += int(np.sum(got.view(np.uint32) != ref.view(np.uint32)))
        assert e <= FP32_REL_TOL, (name, e)
    if check_full_cast and w.n:
        assert torch.equal(r.dev.p16[:w.n].view(torch.int16), r.dev.p32[:w.n].half().view(torch.int16))
    assert r.dev.guard_intact(), "a kernel stored outside the shard's arrays (arena canary changed)"
    del dsrcs
    return {"gen_s": t1 - t0, "step_s": t2 - t1}


# ---- gradient accumulation (fp32 partition) ---------------------------------------

def exact_units32(grad32: np.ndarray) -> Optional[int]:
    """sum of squares in 2^-48 units of fp32 values that are multiples of
    2^-24 below 2^24 (the accumulation domain), as a Python integer: with
    a = x * 2^24 (an integer below 2^48) the square is a^2 units; a is split
    into 16-bit digits so that every partial product sum fits int64.  None
    if some value is off that grid."""
    total = 0
    m = (1 << 16) - 1
    for lo in range(0, grad32.size, 1 << 20):
        x = grad32[lo:lo + (1 << 20)].astype(np.float64)
        a = x * 2.0 ** 24
        if not np.all(np.floor(a) == a) or not np.all(np.abs(a) < 2.0 ** 48):
            return None
        a = np.abs(a).astype(np.int64)
        a0, a1, a2 = a & m, (a >> 16) & m, a >> 32
        sq = lambda u, v: int((u * v).sum())
        total += (sq(a0, a0) + (2 * sq(a0, a1) << 16) + ((sq(a1, a1) + 2 * sq(a0, a2)) << 32)
                  + (2 * sq(a1, a2) << 48) + (sq(a2, a2) << 64))
    return total


@dataclass
class AccumRun:
    w: shardgen.Workload
    micro: int
    sample: Optional[np.ndarray] = None
    dev: Z.AccumStep = None
    st: O.OracleState = None
    hp_o: O.OracleHParams = None
    hp_d: Z.HParams = None
    p16: np.ndarray = None
    p32: np.ndarray = None
    m32: np.ndarray = None
    v32: np.ndarray = None
    k: int = 0
    stats: dict = field(default_factory=lambda: {"fp32_not_bitwise": 0, "fp32_max_rel": 0.0})

    @property
    def n(self) -> int:
        return self.w.n

    def idx(self) -> np.ndarray:
        return np.arange(self.n) if self.sample is None else self.sample


def start_accum(w: shardgen.Workload, micro: int, sample: Optional[int] = None, seed: int = 78,
                fused: bool = True, any_order: bool = True) -> AccumRun:
    r = AccumRun(w, micro)
    n = w.n
    if sample is not None and sample < n:
        rng = np.random.default_rng(seed)
        edges = []
        for _, _, do, c in w.layout.segments:
            edges += [do, do + 1, do + c - 1, do + c - 2]
        edges += list(range(min(n, 64))) + list(range(max(0, n - 64), n))
        r.sample = np.unique(np.clip(np.concatenate([rng.integers(0, n, sample), np.array(edges)]), 0, n - 1))
    p32 = shardgen.master_params(w)
    r.dev = Z.AccumStep(n, fused=fused, any_order=any_order)
    if n:
        r.dev.p32.copy_(torch.from_numpy(p32))
        r.dev.p16.copy_(torch.from_numpy(shardgen.to_f16_bits(p32).view(np.float16)))
    r.dev.init_state(w.scale0)
    i = r.idx()
    r.p32 = np.ascontiguousarray(p32[i])
    r.p16 = shardgen.to_f16_bits(r.p32)
    r.m32 = np.zeros_like(r.p32)
    r.v32 = np.zeros_like(r.p32)
    r.st = O.new_state(w.scale0)
    r.hp_o = oracle_hparams(w.hp)
    r.hp_d = device_hparams(w.hp)
    return r


def step_accum(r: AccumRun, check: bool = True, exact: bool = True) -> None:
    """One optimizer step of r.micro micro-batches on both sides."""
    r.k += 1
    w = r.w
    srcs_all, plans, keep = [], [], []
    for j in range(r.micro):
        gpart = shardgen.grad_partition(w, (r.k - 1) * r.micro + j + 1, r.st.loss_scale)
        srcs = shardgen.source_tensors(w.layout, gpart)
        del gpart
        srcs_all.append(srcs)
        dsrcs = [to_dev16(s) for s in srcs]
        kept, buckets = r.dev.plan(dsrcs, w.layout.segments, w.bucket_elems)
        keep.append(kept)
        plans.append(buckets)
    log(f"{w.name} n={w.n} accum step {r.k}: {r.micro} micro-batches, fused={r.dev.fused}")
    r.dev.step(plans, r.hp_d)
    grad = np.zeros(w.n, np.float32)
    for j, srcs in enumerate(srcs_all):
        O.flatten(srcs, w.layout.segments, grad, accumulate=(j > 0))
    sumsq, ovf = O.norm_overflow_f32(grad)
    O.decide(r.st, r.hp_o, sumsq, ovf)
    i = r.idx()
    O.adam_update_f32(r.st, r.p16, r.p32, r.m32, r.v32, np.ascontiguousarray(grad[i]))
    torch.cuda.synchronize()
    log(f"{w.name} accum step {r.k}: gpu done, overflow={ovf} norm={r.st.grad_norm:.6g}")
    if not check:
        return
    compare_state(r.dev.read_state(), r.st, exact_units32(grad) if (exact and not ovf) else None)
    assert same_floats32(r.dev.grad32[:w.n].cpu().numpy(), grad), "accumulated gradient differs"
    it = torch.from_numpy(i).cuda()
    d16 = bits16(r.dev.p16[it])
    assert np.array_equal(d16, r.p16), f"p16 differs at {int(np.sum(d16 != r.p16))} elements"
    for name, dt, ref in (("p32", r.dev.p32, r.p32), ("m32", r.dev.m32, r.m32), ("v32", r.dev.v32, r.v32)):
        got = dt[it].cpu().numpy()
        e = rel_err(got, ref)
        r.stats["fp32_max_rel"] = max(r.stats["fp32_max_rel"], e)
        r.stats["fp32_not_bitwise"] += int(np.sum(got.view(np.uint32) != ref.view(np.uint32)))
        assert e <= FP32_REL_TOL, (name, e)
    if w.n:
        assert torch.equal(r.dev.p16[:w.n].view(torch.int16), r.dev.p32[:w.n].half().view(torch.int16))
    assert r.dev.guard_intact(), "a kernel stored outside the shard's arrays (arena canary changed)"
    del keep
