"""ShardStep and AccumStep: the C-ABI calls of one ZeRO shard step, wired to
torch-owned device buffers.  Allocation and call order only; the arithmetic is
in the HIP kernels behind the C ABI.

One data-parallel rank owns n parameters of the flat model state (ZeRO paper
card, "Method").  For them it keeps, index-aligned and contiguous: the fp16
parameter copy, the flat fp16 gradient partition, and the fp32 master
parameters, momentum and variance (16 bytes per parameter, "Bottleneck"),
plus the 128-byte step state and the reduction workspace.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

from . import _lib as Z


def host_f32(n: int, huge_pages: bool = True):
    """A zeroed float32 host tensor of n elements.  With huge_pages, it is backed
    by an anonymous mapping aligned to 2 MiB and marked for transparent huge
    pages before first touch (Linux), so streaming it takes one TLB entry and
    no prefetcher stop per 2 MiB instead of per 4 KiB; where that is not
    available, an ordinary torch tensor."""
    import mmap

    import torch
    nbytes = max(1, n) * 4
    if not huge_pages or not hasattr(mmap, "MADV_HUGEPAGE"):
        return torch.zeros(max(1, n), dtype=torch.float32)
    huge = 2 << 20
    m = mmap.mmap(-1, nbytes + huge, flags=mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS)
    base = C.addressof(C.c_char.from_buffer(m))
    skip = (-base) % huge
    try:
        m.madvise(mmap.MADV_HUGEPAGE)
    except OSError:
        pass                                      # huge pages disabled: 4 KiB pages, same contents
    view = memoryview(m)[skip:skip + nbytes]
    t = torch.frombuffer(view, dtype=torch.float32)  # zero-filled by the kernel on first touch
    t._zero_mapping = (m, view)                       # keeps the mapping alive with the tensor
    return t


ARENA_ALIGN = 2 << 20      # every array starts at a 2 MiB boundary of the device address space ...
ARENA_STAGGER = 64 << 10   # ... plus 64 KiB times its index in the arena
ARENA_CANARY = 0xA5        # the byte every gap of the arena holds


class StateArena:
    """The flat per-parameter arrays of a shard, carved out of ONE device
    allocation.  specs is a sequence of (name, numel, torch dtype); array k
    starts at a 2 MiB-aligned device address plus k * 64 KiB, the arrays
    follow each other in the given order, each zero-filled, and `arrays` maps
    each name to its tensor view (the views keep the allocation alive).

    Why: the update streams all of these arrays at once, front by front.  On
    MI355X the same Adam launch ran 1.4-3% faster on the gpt2 shard and 4-5%
    faster on the 1T rank in this layout than on separate allocations, and
    slower with no stagger or with a stagger of 16 KiB or 512 KiB (HIP events,
    two boxes).

    Every byte outside the arrays -- at least 2 MiB before the first, at least
    64 KiB between two, and the tail -- holds ARENA_CANARY, so a kernel that
    stores past either end of an array changes a gap; `intact()` checks them
    all (one device reduction and one host read)."""

    def __init__(self, device, specs, canary: int = ARENA_CANARY):
        import torch
        layout, end = [], ARENA_ALIGN                # the first array starts one alignment in
        for k, (_, numel, dtype) in enumerate(specs):
            size = max(1, int(numel)) * torch.empty((), dtype=dtype).element_size()
            start = -(-end // ARENA_ALIGN) * ARENA_ALIGN + k * ARENA_STAGGER
            layout.append((start, size))
            end = start + size
        self.canary = int(canary)
        self.tensor = torch.full((end + 2 * ARENA_ALIGN,), self.canary, dtype=torch.uint8, device=device)
        skip = (-self.tensor.data_ptr()) % ARENA_ALIGN
        self.arrays = {}
        self.gaps = []
        pos = 0
        for (name, _, dtype), (start, size) in zip(specs, layout):
            lo = skip + start
            self.gaps.append((pos, lo))
            view = self.tensor[lo:lo + size]
            view.zero_()
            self.arrays[name] = view.view(dtype)
            pos = lo + size
        self.gaps.append((pos, self.tensor.numel()))

    def intact(self) -> bool:
        """True if every gap still holds the canary byte (synchronises)."""
        import torch
        bad = torch.stack([(self.tensor[lo:hi] != self.canary).any() for lo, hi in self.gaps])
        return not bool(bad.any().item())


def _segments(sources, segments, fn):
    """(tensor index, src_off, dst_off, count) -> ctypes segments, with every
    source range checked against its tensor on the host."""
    for t, so, do, c in segments:
        if so < 0 or c < 0 or so + c > sources[t].numel():
            raise ValueError(f"{fn}: segment ({t}, {so}, {do}, {c}) reads past its source tensor "
                             f"of {sources[t].numel()} elements")
    return Z.make_segments([(sources[t].data_ptr(), so, do, c) for t, so, do, c in segments])


class ShardStep:
    """fused=False: flatten, then the standalone exact-norm pass over the
    partition.  fused=True: the flatten computes the exact-norm partials while
    it copies and a decide-only pass folds them (no second read of the
    partition).  Both take bit-identical decisions.  any_order=True flattens
    all buckets of a step in one zero_flatten_buckets call (consecutive
    buckets overlap on the GPU); False issues one ordered call per bucket.
    The arrays (p32, m32, v32, grad16, p16 and state) are fixed for the
    object's life: write into them in place; the calls use the addresses
    taken when it was made."""

    def __init__(self, n: int, device="cuda", fused: bool = False, extra=(), any_order: bool = True):
        """extra: further (name, numel, dtype) arrays placed in the same arena
        after the five of the step (attributes of the same names)."""
        import torch
        self.n = int(n)
        alloc = max(1, self.n)
        self.device = torch.device(device)
        f32, f16 = torch.float32, torch.float16
        self.arena = StateArena(self.device, [("p32", alloc, f32), ("m32", alloc, f32), ("v32", alloc, f32),
                                              ("grad16", alloc, f16), ("p16", alloc, f16), *extra])
        for name, t in self.arena.arrays.items():
            setattr(self, name, t)
        self.state = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device=self.device)
        # The arrays never move: their addresses, taken once (the binding
        # passes integer addresses through without checking a tensor again,
        # which is most of a call's host time on a small shard).
        self._addr = {name: t.data_ptr() for name, t in self.arena.arrays.items()}
        self._addr["state"] = self.state.data_ptr()
        ws = Z.zero_norm_workspace_bytes(self.n)
        self.workspace = torch.empty(max(16, ws), dtype=torch.uint8, device=self.device)
        self._buckets = Z.BucketPlan([])
        self._sources: Sequence = ()
        self.fused = bool(fused)
        self.any_order = bool(any_order)
        self.partials = None            # fused form: one 16-byte partial per flatten workgroup
        self.partial_offsets: List[int] = []
        self.partial_count = 0
        self.decide_ws = None

    def __setattr__(self, name, value):
        # An array whose address the calls hold cannot be rebound: the calls
        # would go on using the old one.
        if name in self.__dict__.get("_addr", ()):
            raise AttributeError(f"{type(self).__name__}.{name} is fixed for the object's life (the calls use "
                                 f"its address); write into it in place")
        object.__setattr__(self, name, value)

    # ---- set-up ----------------------------------------------------------------
    @property
    def buckets(self) -> "Z.BucketPlan":
        """The step's buckets: a BucketPlan (assign one, or (segments, count)
        pairs, which are turned into one)."""
        return self._buckets

    @buckets.setter
    def buckets(self, plan) -> None:
        self._buckets = plan if isinstance(plan, Z.BucketPlan) else Z.BucketPlan(plan)

    def init_state(self, initial_scale: float) -> None:
        Z.zero_step_state_init(self.state, initial_scale)

    def set_segments(self, sources: Sequence, segments: Sequence[Tuple[int, int, int, int]],
                     bucket_elems: int = 0) -> None:
        """sources: device fp16 tensors; segments: (tensor index, src_off,
        dst_off, count).  With bucket_elems > 0 the partition is flattened in
        windows of that many destination elements."""
        self._sources = list(sources)                  # keep the tensors alive
        segs, nsegs = _segments(self._sources, segments, "ShardStep.set_segments")
        if bucket_elems and bucket_elems < self.n:
            self.buckets = [Z.zero_bucket_segments(segs, nsegs, b, min(self.n, b + bucket_elems))
                            for b in range(0, self.n, bucket_elems)]
        else:
            self.buckets = [(segs, nsegs)]
        if self.fused:
            self._plan_partials()

    def _plan_partials(self) -> None:
        import torch
        offsets, total = [], 0
        for segs, nsegs in self.buckets:
            offsets.append(total)
            total += Z.zero_flatten_norm_partials(segs, nsegs)
        self.partial_offsets, self.partial_count = offsets, total
        need = max(1, total) * Z.NORM_PARTIAL_BYTES
        if self.partials is None or self.partials.numel() < need:
            self.partials = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = max(16, Z.zero_decide_workspace_bytes(total))
        if self.decide_ws is None or self.decide_ws.numel() < ws:
            self.decide_ws = torch.empty(ws, dtype=torch.uint8, device=self.device)

    # ---- the step ---------------------------------------------------------------
    def flatten(self) -> None:
        if self.any_order:
            Z.zero_flatten_buckets(self.buckets, self._addr["grad16"], self.n, Z.ZERO_F16, False)
            return
        for segs, nsegs in self.buckets:
            Z.zero_flatten_bucket(segs, nsegs, self._addr["grad16"], self.n, Z.ZERO_F16, False)

    def norm_overflow(self, hp: Z.HParams) -> None:
        Z.zero_shard_norm_overflow(self._addr["grad16"], self.n, hp, self._addr["state"], self.workspace)

    def adam(self) -> None:
        a = self._addr
        Z.zero_shard_adam_step(a["p16"], a["p32"], a["m32"], a["v32"], a["grad16"], self.n, a["state"])

    def flatten_norm(self) -> None:
        if self.any_order:
            Z.zero_flatten_buckets(self.buckets, self._addr["grad16"], self.n, Z.ZERO_F16, False, self.partials)
            return
        for (segs, nsegs), off in zip(self.buckets, self.partial_offsets):
            Z.zero_flatten_norm_bucket(segs, nsegs, self._addr["grad16"], self.partials, self.n, False, off)

    def decide(self, hp: Z.HParams) -> None:
        Z.zero_shard_decide(self.partials, self.partial_count, hp, self._addr["state"], self.decide_ws)

    def step(self, hp: Z.HParams) -> None:
        if self.fused:
            self.flatten_norm()
            self.decide(hp)
        else:
            self.flatten()
            self.norm_overflow(hp)
        self.adam()

    def guard_intact(self) -> bool:
        """True if no kernel has stored outside the shard's arrays (the
        arena's canary gaps are unchanged); synchronises."""
        return self.arena.intact()

    def read_state(self) -> Z.StepState:
        return Z.read_state(self.state)


class AccumStep:
    """The gradient-accumulation form of the step: K micro-batches of per-layer
    fp16 gradients are added into an fp32 partition, then the fp32 reduction
    and the update reading the fp32 gradient run (the DeepSpeed article leaves
    gradient accumulation to the library).  fused=True computes the
    exact-norm partials in the last micro-batch's flatten and folds them with
    the decide-only pass; fused=False runs the standalone fp32 reduction.
    Both take bit-identical decisions."""

    def __init__(self, n: int, device="cuda", fused: bool = True, any_order: bool = True):
        import torch
        self.n = int(n)
        alloc = max(1, self.n)
        self.device = torch.device(device)
        f32 = torch.float32
        self.arena = StateArena(self.device, [("p32", alloc, f32), ("m32", alloc, f32), ("v32", alloc, f32),
                                              ("grad32", alloc, f32), ("p16", alloc, torch.float16)])
        for name, t in self.arena.arrays.items():
            setattr(self, name, t)
        self.state = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device=self.device)
        ws = Z.zero_norm_workspace_bytes(self.n)
        self.workspace = torch.empty(max(16, ws), dtype=torch.uint8, device=self.device)
        self.fused = bool(fused)
        self.any_order = bool(any_order)
        self.partials = None
        self.decide_ws = None
        self.partial_count = 0
        self.partial_offsets: List[int] = []

    def init_state(self, initial_scale: float) -> None:
        Z.zero_step_state_init(self.state, initial_scale)

    def plan(self, sources: Sequence, segments: Sequence[Tuple[int, int, int, int]], bucket_elems: int = 0):
        """One micro-batch's segment plan: (kept sources, BucketPlan)."""
        sources = list(sources)
        segs, nsegs = _segments(sources, segments, "AccumStep.plan")
        if bucket_elems and bucket_elems < self.n:
            buckets = [Z.zero_bucket_segments(segs, nsegs, b, min(self.n, b + bucket_elems))
                       for b in range(0, self.n, bucket_elems)]
        else:
            buckets = [(segs, nsegs)]
        buckets = Z.BucketPlan(buckets)
        if self.fused:
            self._size_partials(buckets)
        return sources, buckets

    def _size_partials(self, buckets) -> None:
        import torch
        offsets, total = [], 0
        for segs, nsegs in buckets:
            offsets.append(total)
            total += Z.zero_flatten_norm_partials(segs, nsegs)
        self.partial_offsets, self.partial_count = offsets, total
        need = max(1, total) * Z.NORM_PARTIAL_BYTES
        if self.partials is None or self.partials.numel() < need:
            self.partials = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = max(16, Z.zero_decide_workspace_bytes(total))
        if self.decide_ws is None or self.decide_ws.numel() < ws:
            self.decide_ws = torch.empty(ws, dtype=torch.uint8, device=self.device)

    def accumulate(self, buckets, first: bool) -> None:
        """Widen (first micro-batch) or add one micro-batch into grad32."""
        if self.any_order:
            Z.zero_flatten_buckets(buckets, self.grad32, self.n, Z.ZERO_F32, not first)
            return
        for segs, nsegs in buckets:
            Z.zero_flatten_bucket(segs, nsegs, self.grad32, self.n, Z.ZERO_F32, not first)

    def accumulate_norm(self, buckets, first: bool) -> None:
        """The last micro-batch's flatten, computing the exact-norm partials of
        the finished fp32 partition (requires fused=True)."""
        if self.partial_count != sum(Z.zero_flatten_norm_partials(s, k) for s, k in buckets):
            self._size_partials(buckets)
        if self.any_order:
            Z.zero_flatten_buckets(buckets, self.grad32, self.n, Z.ZERO_F32, not first, self.partials)
            return
        for (segs, nsegs), off in zip(buckets, self.partial_offsets):
            Z.zero_flatten_norm_bucket_f32(segs, nsegs, self.grad32, self.partials, self.n, not first, off)

    def norm_overflow(self, hp: Z.HParams) -> None:
        Z.zero_shard_norm_overflow_f32(self.grad32, self.n, hp, self.state, self.workspace)

    def decide(self, hp: Z.HParams) -> None:
        Z.zero_shard_decide_f32(self.partials, self.partial_count, self.grad32, self.n, hp, self.state,
                                self.decide_ws)

    def adam(self) -> None:
        Z.zero_shard_adam_step_f32(self.p16, self.p32, self.m32, self.v32, self.grad32, self.n, self.state)

    def step(self, micro_batches, hp: Z.HParams) -> None:
        """micro_batches: bucket plans from plan(), in accumulation order."""
        k = len(micro_batches)
        for i, buckets in enumerate(micro_batches):
            if self.fused and i == k - 1:
                self.accumulate_norm(buckets, first=(i == 0))
            else:
                self.accumulate(buckets, first=(i == 0))
        if self.fused:
            self.decide(hp)
        else:
            self.norm_overflow(hp)
        self.adam()

    def guard_intact(self) -> bool:
        """True if no kernel has stored outside the shard's arrays (the
        arena's canary gaps are unchanged); synchronises."""
        return self.arena.intact()

    def read_state(self) -> Z.StepState:
        return Z.read_state(self.state)


class OneBitStep(ShardStep):
    """1-bit Adam on the shard (the DeepSpeed article; Tang et al. 2021,
    Algorithm 1): the first `warmup` applied steps are the ordinary update,
    which also builds the variance; after them the variance is frozen and each
    step runs the compression stage.  The flatten with exact-norm partials and
    the decision are the same in both stages, and the device picks the stage
    from its own applied-step count (zero_onebit_step), so a step never reads
    the state back and a captured step replays correctly on both sides of the
    hand-over."""

    def __init__(self, n: int, warmup: int, device="cuda"):
        import torch
        alloc = max(1, int(n))
        super().__init__(n, device=device, fused=True,
                         extra=[("err_w", alloc, torch.float32), ("err_s", alloc, torch.float32),
                                ("bits_w", (alloc + 7) // 8, torch.uint8), ("bits_s", (alloc + 7) // 8, torch.uint8)])
        self.warmup = int(warmup)
        self.onebit = torch.zeros(Z.ONEBIT_STATE_BYTES, dtype=torch.uint8, device=self.device)
        self.onebit_ws = torch.empty(max(256, Z.zero_onebit_workspace_bytes(self.n)), dtype=torch.uint8,
                                     device=self.device)

    def init_state(self, initial_scale: float) -> None:
        super().init_state(initial_scale)
        Z.zero_onebit_state_init(self.onebit)

    def compressing(self) -> bool:
        """Whether the next step runs the compression stage (reads the state
        back: a synchronisation, for callers outside the step)."""
        return int(self.read_state().step) >= self.warmup

    def update(self) -> None:
        """The update of a decided step: the ordinary one during the warm-up,
        the compression stage after it (the device chooses)."""
        Z.zero_onebit_step(self.p16, self.p32, self.m32, self.v32, self.err_w, self.err_s, self.grad16, self.n,
                           self.bits_w, self.bits_s, self.state, self.onebit, self.warmup, self.onebit_ws)

    def step(self, hp: Z.HParams) -> None:
        self.flatten_norm()
        self.decide(hp)
        self.update()

    def read_onebit(self) -> Z.OneBitState:
        return Z.read_onebit_state(self.onebit)


class HostContext:
    """Owns a zero_host_ctx_t (the host step's worker pool)."""

    def __init__(self, threads: int = 0):
        self.ptr = Z.zero_host_create(threads)
        self._destroy = Z.lib().zero_host_destroy  # the C function itself: still callable at interpreter exit

    @property
    def threads(self) -> int:
        return Z.zero_host_threads(self.ptr)

    def close(self) -> None:
        if self.ptr:
            self._destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        self.close()


class OffloadStep:
    """The ZeRO-Offload form of the step (the DeepSpeed article: ZeRO-2 plus CPU
    memory).  On the device: the per-layer fp16 gradients, the flat fp16
    gradient partition the flatten packs them into, and the fp16 parameters.
    In host memory: the fp32 master parameters, momentum and variance, the
    pinned staging copies of the fp16 gradient and parameters, and the step
    state (pinned).

    device_decides=True (default): the flatten computes the exact-norm
    partials and the device decides (a few microseconds), so the CPU can
    update each gradient chunk as soon as it lands.  device_decides=False: the
    CPU reduces the gradient and decides.  Both decide bit-identically.
    The defaults (transfer chunks of at most 16M elements, ramped at both
    ends by the library; all CPUs but one) were the fastest measured on the
    gpt2 shard.  huge_pages: back the host fp32 state
    with transparent huge pages (host_f32)."""

    def __init__(self, n: int, threads: Optional[int] = None, chunk_elems: int = 1 << 24, device="cuda",
                 device_decides: bool = True, huge_pages: bool = True):
        import os
        import torch
        self.n = int(n)
        alloc = max(1, self.n)
        self.device = torch.device(device)
        if threads is None:          # every CPU but one, which the HIP runtime's copy/event threads use
            threads = max(1, len(os.sched_getaffinity(0)) - 1)
        self.ctx = HostContext(threads)
        self.chunk = int(chunk_elems)
        self.device_decides = bool(device_decides)
        self.grad16 = torch.zeros(alloc, dtype=torch.float16, device=self.device)
        self.p16 = torch.zeros(alloc, dtype=torch.float16, device=self.device)
        self.host_grad16 = torch.zeros(alloc, dtype=torch.float16, pin_memory=True)
        self.host_p16 = torch.zeros(alloc, dtype=torch.float16, pin_memory=True)
        self.p32 = host_f32(alloc, huge_pages)
        self.m32 = host_f32(alloc, huge_pages)
        self.v32 = host_f32(alloc, huge_pages)
        self.state = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, pin_memory=True)
        self.dev_state = torch.zeros(Z.STATE_BYTES, dtype=torch.uint8, device=self.device)
        self.buckets: List[Tuple[object, int]] = []
        self._sources: Sequence = ()
        self.partials = None
        self.partial_offsets: List[int] = []
        self.partial_count = 0
        self.decide_ws = None

    def _host_state(self) -> Z.StepState:
        return Z.StepState.from_address(self.state.data_ptr())

    def init_state(self, initial_scale: float) -> None:
        Z.zero_host_state_init(self._host_state(), initial_scale)
        if self.device_decides:
            Z.zero_step_state_init(self.dev_state, initial_scale)

    def set_segments(self, sources: Sequence, segments: Sequence[Tuple[int, int, int, int]],
                     bucket_elems: int = 0) -> None:
        import torch
        self._sources = list(sources)
        segs, nsegs = _segments(self._sources, segments, "OffloadStep.set_segments")
        if bucket_elems and bucket_elems < self.n:
            self.buckets = [Z.zero_bucket_segments(segs, nsegs, b, min(self.n, b + bucket_elems))
                            for b in range(0, self.n, bucket_elems)]
        else:
            self.buckets = [(segs, nsegs)]
        if self.device_decides:
            offsets, total = [], 0
            for sg, k in self.buckets:
                offsets.append(total)
                total += Z.zero_flatten_norm_partials(sg, k)
            self.partial_offsets, self.partial_count = offsets, total
            need = max(1, total) * Z.NORM_PARTIAL_BYTES
            if self.partials is None or self.partials.numel() < need:
                self.partials = torch.empty(need, dtype=torch.uint8, device=self.device)
            ws = max(16, Z.zero_decide_workspace_bytes(total))
            if self.decide_ws is None or self.decide_ws.numel() < ws:
                self.decide_ws = torch.empty(ws, dtype=torch.uint8, device=self.device)

    def flatten(self, hp: Z.HParams) -> None:
        if self.device_decides:
            for (sg, k), off in zip(self.buckets, self.partial_offsets):
                Z.zero_flatten_norm_bucket(sg, k, self.grad16, self.partials, self.n, False, off)
            Z.zero_shard_decide(self.partials, self.partial_count, hp, self.dev_state, self.decide_ws)
        else:
            for sg, k in self.buckets:
                Z.zero_flatten_bucket(sg, k, self.grad16, self.n, Z.ZERO_F16, False)

    def offload(self, hp: Z.HParams) -> None:
        Z.zero_offload_step(self.ctx.ptr, self.grad16, self.p16, self.host_grad16, self.host_p16, self.p32,
                            self.m32, self.v32, self.n, hp, self.state.data_ptr(),
                            self.dev_state if self.device_decides else None, self.chunk)

    def step(self, hp: Z.HParams) -> None:
        self.flatten(hp)
        self.offload(hp)

    def read_state(self) -> Z.StepState:
        return Z.StepState.from_buffer_copy(self.state.numpy().tobytes())


def hparams(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=1.0,
            backoff=0.5, growth=2.0, min_scale=1.0, growth_interval=20) -> Z.HParams:
    return Z.HParams(lr, beta1, beta2, eps, weight_decay, max_grad_norm, backoff, growth, min_scale,
                     growth_interval, 0)
