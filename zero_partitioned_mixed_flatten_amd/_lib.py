"""ctypes binding of libzero_mi355x.so: one Python function per C entry point,
with the same names.  Argument marshalling only -- torch tensors supply device
memory and the current HIP stream; every step of the path runs in the HIP
kernels behind the C ABI.  There is no fallback: if the library is missing
the import fails loudly."""
from __future__ import annotations

import ctypes as C
import os
from typing import Iterable, List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero_mi355x.so")

ZERO_OK, ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE, ZERO_EHIP, ZERO_ENOTSUP, ZERO_ENOMEM = 0, -1, -2, -3, -4, -5, -6
ZERO_F16, ZERO_F32 = 1, 2

# Every function the public header declares (checked against the header by a test).
EXPORTS = ("zero_status_string", "zero_state_bytes", "zero_bucket_segments", "zero_step_state_init",
           "zero_flatten_bucket", "zero_norm_workspace_bytes", "zero_shard_norm_overflow",
           "zero_shard_adam_step", "zero_stream_copy", "zero_flatten_norm_partials", "zero_flatten_norm_bucket",
           "zero_decide_workspace_bytes", "zero_shard_decide", "zero_flatten_norm_bucket_f32", "zero_flatten_buckets",
           "zero_shard_norm_overflow_f32", "zero_shard_adam_step_f32", "zero_host_create", "zero_host_destroy",
           "zero_host_threads", "zero_host_state_init", "zero_host_norm_overflow", "zero_host_adam_step",
           "zero_offload_step", "zero_host_stream_copy", "zero_onebit_state_init", "zero_onebit_workspace_bytes",
           "zero_onebit_step", "zero_shard_norm_overflow_noalloc", "zero_shard_decide_f32")
NORM_PARTIAL_BYTES = 16


class ZeroError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {code} ({text})")
        self.code = code


class Segment(C.Structure):
    _fields_ = [("src", C.c_void_p), ("src_off", C.c_uint64), ("dst_off", C.c_uint64),
                ("count", C.c_uint64)]


class HParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double),
                ("weight_decay", C.c_double), ("max_grad_norm", C.c_double), ("backoff", C.c_double),
                ("growth", C.c_double), ("min_scale", C.c_double), ("growth_interval", C.c_int32),
                ("reserved", C.c_int32)]


class StepState(C.Structure):
    _fields_ = [("loss_scale", C.c_double), ("beta1_pow", C.c_double), ("beta2_pow", C.c_double),
                ("step", C.c_int64), ("good_steps", C.c_int32), ("skipped_total", C.c_int32),
                ("sumsq", C.c_double), ("grad_norm", C.c_double), ("overflow", C.c_int32),
                ("skip", C.c_int32), ("gmul", C.c_float), ("bc1", C.c_float), ("bc2", C.c_float),
                ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("omb1", C.c_float),
                ("omb2", C.c_float), ("eps", C.c_float), ("wd", C.c_float), ("done_blocks", C.c_uint32),
                ("wide_pending", C.c_uint32), ("sumsq_units", C.c_uint64 * 2)]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_ if name != "sumsq_units"}
        d["sumsq_units"] = (int(self.sumsq_units[1]) << 64) | int(self.sumsq_units[0])
        return d


class OneBitState(C.Structure):
    _fields_ = [("scale_w", C.c_float), ("scale_s", C.c_float), ("sumsq_w", C.c_double), ("sumsq_s", C.c_double),
                ("qexp_w", C.c_int32), ("qexp_s", C.c_int32), ("done_blocks", C.c_uint32),
                ("wide_pending", C.c_uint32), ("units_w", C.c_uint64 * 2), ("units_s", C.c_uint64 * 2)]

    def units(self, which: str) -> int:
        u = getattr(self, f"units_{which}")
        return (int(u[1]) << 64) | int(u[0])


STATE_BYTES = C.sizeof(StepState)
ONEBIT_STATE_BYTES = C.sizeof(OneBitState)
assert STATE_BYTES == 128 and C.sizeof(Segment) == 32 and C.sizeof(HParams) == 80 and ONEBIT_STATE_BYTES == 72

_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        # torch first: the library then binds to the HIP runtime torch has
        # already loaded (the same soname), so one runtime serves both;
        # loaded the other way round, torch's tensors and this library's
        # launches would live in two runtimes and the device calls fail.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        vp, u64, u32, i32 = C.c_void_p, C.c_uint64, C.c_uint32, C.c_int
        L.zero_status_string.argtypes = [i32]
        L.zero_status_string.restype = C.c_char_p
        L.zero_state_bytes.argtypes = [u64, u32, u32, i32, C.POINTER(u64)]
        L.zero_bucket_segments.argtypes = [C.POINTER(Segment), u32, u64, u64, C.POINTER(Segment), u32,
                                           C.POINTER(u32)]
        L.zero_step_state_init.argtypes = [vp, C.c_double, vp]
        L.zero_flatten_bucket.argtypes = [C.POINTER(Segment), u32, vp, u64, i32, i32, vp]
        L.zero_norm_workspace_bytes.argtypes = [u64]
        L.zero_norm_workspace_bytes.restype = C.c_size_t
        L.zero_shard_norm_overflow.argtypes = [vp, u64, C.POINTER(HParams), vp, vp, C.c_size_t, vp]
        L.zero_shard_norm_overflow_f32.argtypes = [vp, u64, C.POINTER(HParams), vp, vp, C.c_size_t, vp]
        L.zero_shard_norm_overflow_noalloc.argtypes = [vp, u64, C.POINTER(HParams), vp, vp]
        L.zero_shard_adam_step.argtypes = [vp, vp, vp, vp, vp, u64, vp, vp]
        L.zero_shard_adam_step_f32.argtypes = [vp, vp, vp, vp, vp, u64, vp, vp]
        L.zero_stream_copy.argtypes = [vp, vp, u64, vp]
        L.zero_flatten_norm_partials.argtypes = [C.POINTER(Segment), u32]
        L.zero_flatten_norm_partials.restype = u64
        L.zero_flatten_norm_bucket.argtypes = [C.POINTER(Segment), u32, vp, u64, i32, vp, u64, vp]
        L.zero_flatten_norm_bucket_f32.argtypes = [C.POINTER(Segment), u32, vp, u64, i32, vp, u64, vp]
        L.zero_flatten_buckets.argtypes = [C.POINTER(Segment), C.POINTER(u32), u32, vp, u64, i32, i32, vp, u64, vp]
        L.zero_decide_workspace_bytes.argtypes = [u64]
        L.zero_decide_workspace_bytes.restype = C.c_size_t
        L.zero_shard_decide.argtypes = [vp, u64, C.POINTER(HParams), vp, vp, C.c_size_t, vp]
        L.zero_shard_decide_f32.argtypes = [vp, u64, vp, u64, C.POINTER(HParams), vp, vp, C.c_size_t, vp]
        L.zero_host_create.argtypes = [i32, C.POINTER(vp)]
        L.zero_host_destroy.argtypes = [vp]
        L.zero_host_destroy.restype = None
        L.zero_host_threads.argtypes = [vp]
        L.zero_host_state_init.argtypes = [C.POINTER(StepState), C.c_double]
        L.zero_host_norm_overflow.argtypes = [vp, vp, u64, C.POINTER(HParams), C.POINTER(StepState)]
        L.zero_host_adam_step.argtypes = [vp, vp, vp, vp, vp, vp, u64, C.POINTER(StepState)]
        L.zero_offload_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, u64, C.POINTER(HParams), vp, vp, u64, vp]
        L.zero_host_stream_copy.argtypes = [vp, vp, vp, u64]
        L.zero_onebit_state_init.argtypes = [vp, vp]
        L.zero_onebit_workspace_bytes.argtypes = [u64]
        L.zero_onebit_workspace_bytes.restype = C.c_size_t
        L.zero_onebit_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, u64, vp, vp, vp, vp, C.c_int64, vp, C.c_size_t,
                                       vp]
        for name in EXPORTS:
            if name not in ("zero_status_string", "zero_norm_workspace_bytes", "zero_flatten_norm_partials",
                            "zero_decide_workspace_bytes", "zero_host_destroy", "zero_onebit_workspace_bytes"):
                getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != ZERO_OK:
        raise ZeroError(fn, rc, zero_status_string(rc))


_raw_stream = None


def _stream(stream) -> int:
    """The HIP stream handle of `stream`, or of torch's current stream on the
    current device.  The current one is read through torch's raw-handle
    getter where it exists (the same handle as
    torch.cuda.current_stream().cuda_stream, without building a Stream object:
    0.07 against 2.7 us per call, which the launch-bound small shards feel)."""
    global _raw_stream
    import torch
    if stream is not None:
        return int(stream.cuda_stream)
    if _raw_stream is None:
        get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        _raw_stream = (lambda: get(dev())) if get and dev else (lambda: torch.cuda.current_stream().cuda_stream)
    return int(_raw_stream())


def _need(fn: str, t, nbytes: int) -> None:
    """Raise on the host, before any device work, if tensor `t` holds fewer than
    nbytes bytes (the C ABI takes raw pointers and cannot check this itself).
    Raw integer addresses are passed through unchecked."""
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if nbytes > have:
        raise ValueError(f"{fn}: buffer holds {have} bytes, the call would touch {nbytes}")


def _ptr(t, dtype=None) -> int:
    import torch
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


# ---- host-only entry points ---------------------------------------------------

def zero_status_string(code: int) -> str:
    return lib().zero_status_string(code).decode()


def zero_state_bytes(psi: int, nd: int, k: int = 12, stage: int = 3) -> int:
    out = C.c_uint64()
    _check("zero_state_bytes", lib().zero_state_bytes(psi, nd, k, stage, C.byref(out)))
    return out.value


def make_segments(segs: Sequence[Tuple[int, int, int, int]]):
    """(src_device_ptr, src_off, dst_off, count) tuples -> ctypes array."""
    arr = (Segment * max(1, len(segs)))()
    for i, (p, so, do, cnt) in enumerate(segs):
        arr[i] = Segment(p, so, do, cnt)
    return arr, len(segs)


def zero_bucket_segments(segs, nsegs: int, begin: int, end: int):
    """Cut a ctypes Segment array to the destination window [begin, end)."""
    need = C.c_uint32()
    rc = lib().zero_bucket_segments(segs, nsegs, begin, end, None, 0, C.byref(need))
    if rc not in (ZERO_OK, ZERO_ERANGE):
        _check("zero_bucket_segments", rc)
    out = (Segment * max(1, need.value))()
    got = C.c_uint32()
    _check("zero_bucket_segments",
           lib().zero_bucket_segments(segs, nsegs, begin, end, out, need.value, C.byref(got)))
    return out, got.value


class BucketPlan:
    """The buckets of one step as zero_flatten_buckets takes them: every
    bucket's segments in one host array and the per-bucket counts, built once.
    Iterates as the (segments, count) pairs it was made from."""

    def __init__(self, buckets):
        self.parts = [(segs, int(k)) for segs, k in buckets]
        self.nsegs = sum(k for _, k in self.parts)
        self.segs = (Segment * max(1, self.nsegs))()
        size, pos = C.sizeof(Segment), 0
        for segs, k in self.parts:
            if k:
                C.memmove(C.addressof(self.segs) + pos * size, C.addressof(segs), k * size)
            pos += k
        self.counts = (C.c_uint32 * max(1, len(self.parts)))(*[k for _, k in self.parts])

    def __len__(self):
        return len(self.parts)

    def __iter__(self):
        return iter(self.parts)

    def __getitem__(self, i):
        return self.parts[i]

    def partials(self) -> int:
        """Partials the fused form writes for the whole plan."""
        return int(lib().zero_flatten_norm_partials(self.segs, self.nsegs))


def zero_norm_workspace_bytes(n: int) -> int:
    return int(lib().zero_norm_workspace_bytes(n))


# ---- device entry points (asynchronous on the current torch stream) ---------------

def zero_step_state_init(dev_state, initial_scale: float, stream=None) -> None:
    _need("zero_step_state_init", dev_state, STATE_BYTES)
    _check("zero_step_state_init", lib().zero_step_state_init(_ptr(dev_state), initial_scale, _stream(stream)))


def zero_flatten_bucket(segs, nsegs: int, dst, dst_len: Optional[int] = None, dst_dtype: int = ZERO_F16,
                        accumulate: bool = False, stream=None) -> None:
    if dst_len is None:
        dst_len = dst.numel()
    _need("zero_flatten_bucket", dst, dst_len * (4 if dst_dtype == ZERO_F32 else 2))
    _check("zero_flatten_bucket", lib().zero_flatten_bucket(segs, nsegs, _ptr(dst), dst_len, dst_dtype,
                                                            int(bool(accumulate)), _stream(stream)))


def zero_shard_norm_overflow(grad16, n: int, hp: HParams, dev_state, workspace, stream=None) -> None:
    _need("zero_shard_norm_overflow", grad16, 2 * n)
    _need("zero_shard_norm_overflow", dev_state, STATE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_norm_overflow",
           lib().zero_shard_norm_overflow(_ptr(grad16), n, C.byref(hp), _ptr(dev_state), _ptr(workspace),
                                          ws_bytes, _stream(stream)))


def zero_shard_norm_overflow_noalloc(grad16, n: int, hp: HParams, dev_state, stream=None) -> None:
    _need("zero_shard_norm_overflow_noalloc", grad16, 2 * n)
    _need("zero_shard_norm_overflow_noalloc", dev_state, STATE_BYTES)
    _check("zero_shard_norm_overflow_noalloc",
           lib().zero_shard_norm_overflow_noalloc(_ptr(grad16), n, C.byref(hp), _ptr(dev_state), _stream(stream)))


def zero_shard_norm_overflow_f32(grad32, n: int, hp: HParams, dev_state, workspace, stream=None) -> None:
    _need("zero_shard_norm_overflow_f32", grad32, 4 * n)
    _need("zero_shard_norm_overflow_f32", dev_state, STATE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_norm_overflow_f32",
           lib().zero_shard_norm_overflow_f32(_ptr(grad32), n, C.byref(hp), _ptr(dev_state), _ptr(workspace),
                                              ws_bytes, _stream(stream)))


def zero_shard_adam_step(p16, p32, m32, v32, grad16, n: int, dev_state, stream=None) -> None:
    for t, b in ((p16, 2), (p32, 4), (m32, 4), (v32, 4), (grad16, 2)):
        _need("zero_shard_adam_step", t, b * n)
    _need("zero_shard_adam_step", dev_state, STATE_BYTES)
    _check("zero_shard_adam_step",
           lib().zero_shard_adam_step(_ptr(p16), _ptr(p32), _ptr(m32), _ptr(v32), _ptr(grad16), n,
                                      _ptr(dev_state), _stream(stream)))


def zero_shard_adam_step_f32(p16, p32, m32, v32, grad32, n: int, dev_state, stream=None) -> None:
    for t, b in ((p16, 2), (p32, 4), (m32, 4), (v32, 4), (grad32, 4)):
        _need("zero_shard_adam_step_f32", t, b * n)
    _need("zero_shard_adam_step_f32", dev_state, STATE_BYTES)
    _check("zero_shard_adam_step_f32",
           lib().zero_shard_adam_step_f32(_ptr(p16), _ptr(p32), _ptr(m32), _ptr(v32), _ptr(grad32), n,
                                          _ptr(dev_state), _stream(stream)))


def zero_stream_copy(dst, src, nbytes: int, stream=None) -> None:
    _need("zero_stream_copy", dst, nbytes)
    _need("zero_stream_copy", src, nbytes)
    _check("zero_stream_copy", lib().zero_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def zero_flatten_norm_partials(segs, nsegs: int) -> int:
    return int(lib().zero_flatten_norm_partials(segs, nsegs))


def zero_flatten_norm_bucket(segs, nsegs: int, dst, partials, dst_len: Optional[int] = None,
                             accumulate: bool = False, partials_offset: int = 0, stream=None) -> None:
    """Fused fp16 flatten + exact-norm partials; writes them from entry
    `partials_offset` of the uint8 device buffer `partials`."""
    if dst_len is None:
        dst_len = dst.numel()
    _need("zero_flatten_norm_bucket", dst, 2 * dst_len)
    cap = partials.numel() // NORM_PARTIAL_BYTES - partials_offset
    ptr = _ptr(partials) + partials_offset * NORM_PARTIAL_BYTES
    _check("zero_flatten_norm_bucket",
           lib().zero_flatten_norm_bucket(segs, nsegs, _ptr(dst), dst_len, int(bool(accumulate)), ptr, cap,
                                          _stream(stream)))


def zero_flatten_buckets(plan, dst, dst_len: Optional[int] = None, dst_dtype: int = ZERO_F16,
                         accumulate: bool = False, partials=None, partials_offset: int = 0, stream=None) -> None:
    """Every bucket of `plan` (a BucketPlan, or (segments, count) pairs) in one
    call, consecutive buckets overlapping on the GPU; with `partials` (a
    uint8 device buffer) the fused form, writing from entry `partials_offset`."""
    if not isinstance(plan, BucketPlan):
        plan = BucketPlan(plan)
    if dst_len is None:
        dst_len = dst.numel()
    _need("zero_flatten_buckets", dst, dst_len * (4 if dst_dtype == ZERO_F32 else 2))
    ptr, cap = 0, 0
    if partials is not None:
        cap = partials.numel() // NORM_PARTIAL_BYTES - partials_offset
        ptr = _ptr(partials) + partials_offset * NORM_PARTIAL_BYTES
    _check("zero_flatten_buckets",
           lib().zero_flatten_buckets(plan.segs, plan.counts, len(plan), _ptr(dst), dst_len, dst_dtype,
                                      int(bool(accumulate)), ptr, cap, _stream(stream)))


def zero_flatten_norm_bucket_f32(segs, nsegs: int, dst, partials, dst_len: Optional[int] = None,
                                 accumulate: bool = False, partials_offset: int = 0, stream=None) -> None:
    """Fused fp32 flatten (widen or accumulate) + exact-norm partials of the
    values stored; partials as for zero_flatten_norm_bucket."""
    if dst_len is None:
        dst_len = dst.numel()
    _need("zero_flatten_norm_bucket_f32", dst, 4 * dst_len)
    cap = partials.numel() // NORM_PARTIAL_BYTES - partials_offset
    ptr = _ptr(partials) + partials_offset * NORM_PARTIAL_BYTES
    _check("zero_flatten_norm_bucket_f32",
           lib().zero_flatten_norm_bucket_f32(segs, nsegs, _ptr(dst), dst_len, int(bool(accumulate)), ptr, cap,
                                              _stream(stream)))


def zero_decide_workspace_bytes(count: int) -> int:
    return int(lib().zero_decide_workspace_bytes(count))


def zero_shard_decide(partials, count: int, hp: HParams, dev_state, workspace, stream=None) -> None:
    _need("zero_shard_decide", partials, NORM_PARTIAL_BYTES * count)
    _need("zero_shard_decide", dev_state, STATE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_decide",
           lib().zero_shard_decide(_ptr(partials), count, C.byref(hp), _ptr(dev_state), _ptr(workspace), ws_bytes,
                                   _stream(stream)))


def zero_shard_decide_f32(partials, count: int, grad32, n: int, hp: HParams, dev_state, workspace,
                          stream=None) -> None:
    _need("zero_shard_decide_f32", partials, count * NORM_PARTIAL_BYTES)
    _need("zero_shard_decide_f32", grad32, 4 * n)
    _need("zero_shard_decide_f32", dev_state, STATE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_shard_decide_f32",
           lib().zero_shard_decide_f32(_ptr(partials), count, _ptr(grad32), n, C.byref(hp), _ptr(dev_state),
                                       _ptr(workspace), ws_bytes, _stream(stream)))


def read_state(dev_state) -> StepState:
    """Copy a device step state to the host (synchronises the current stream)."""
    raw = dev_state.detach().to("cpu").numpy().tobytes()
    return StepState.from_buffer_copy(raw)


# ---- host step (ZeRO-Offload form) -------------------------------------------------

def _hptr(a) -> int:
    """Host address of a contiguous numpy array or CPU torch tensor (or an int)."""
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    if hasattr(a, "ctypes"):                         # numpy
        if not a.flags.c_contiguous:
            raise ValueError("expected a contiguous array")
        return a.ctypes.data
    if a.is_cuda:
        raise ValueError("expected host memory")
    if not a.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return a.data_ptr()


def zero_host_create(threads: int = 0) -> int:
    out = C.c_void_p()
    _check("zero_host_create", lib().zero_host_create(threads, C.byref(out)))
    return out.value


def zero_host_destroy(ctx: int) -> None:
    lib().zero_host_destroy(ctx)


def zero_host_threads(ctx: int) -> int:
    return int(lib().zero_host_threads(ctx))


def zero_host_state_init(state: StepState, initial_scale: float) -> None:
    _check("zero_host_state_init", lib().zero_host_state_init(C.byref(state), initial_scale))


def _hneed(fn: str, a, nbytes: int) -> None:
    if a is None or isinstance(a, int):
        return
    have = a.nbytes if hasattr(a, "nbytes") and not hasattr(a, "element_size") else a.numel() * a.element_size()
    if nbytes > have:
        raise ValueError(f"{fn}: buffer holds {have} bytes, the call would touch {nbytes}")


def zero_host_norm_overflow(ctx: int, grad16, n: int, hp: HParams, state: StepState) -> None:
    _hneed("zero_host_norm_overflow", grad16, 2 * n)
    _check("zero_host_norm_overflow",
           lib().zero_host_norm_overflow(ctx, _hptr(grad16), n, C.byref(hp), C.byref(state)))


def zero_host_adam_step(ctx: int, p16, p32, m32, v32, grad16, n: int, state: StepState) -> None:
    for a, b in ((p16, 2), (p32, 4), (m32, 4), (v32, 4), (grad16, 2)):
        _hneed("zero_host_adam_step", a, b * n)
    _check("zero_host_adam_step",
           lib().zero_host_adam_step(ctx, _hptr(p16), _hptr(p32), _hptr(m32), _hptr(v32), _hptr(grad16), n,
                                     C.byref(state)))


def zero_offload_step(ctx: int, dev_grad16, dev_p16, host_grad16, host_p16, p32, m32, v32, n: int,
                      hp: Optional[HParams], state, dev_state=None, chunk_elems: int = 1 << 22, stream=None) -> None:
    """state: a host StepState or the host address of one (e.g. a pinned
    128-byte tensor); dev_state: a device state the device has already
    decided on this stream, or None to decide on the CPU."""
    for t, b in ((dev_grad16, 2), (dev_p16, 2), (host_grad16, 2), (host_p16, 2), (p32, 4), (m32, 4), (v32, 4)):
        _need("zero_offload_step", t, b * n)
    _need("zero_offload_step", dev_state, STATE_BYTES)
    if not isinstance(state, StepState):
        _need("zero_offload_step", state, STATE_BYTES)
    st = C.addressof(state) if isinstance(state, StepState) else _hptr(state)
    _check("zero_offload_step",
           lib().zero_offload_step(ctx, _ptr(dev_grad16), _ptr(dev_p16), _hptr(host_grad16), _hptr(host_p16),
                                   _hptr(p32), _hptr(m32), _hptr(v32), n, C.byref(hp) if hp is not None else None,
                                   st, _ptr(dev_state) if dev_state is not None else None, chunk_elems,
                                   _stream(stream)))


def zero_host_stream_copy(ctx: int, dst, src, nbytes: int) -> None:
    _hneed("zero_host_stream_copy", dst, nbytes)
    _hneed("zero_host_stream_copy", src, nbytes)
    _check("zero_host_stream_copy", lib().zero_host_stream_copy(ctx, _hptr(dst), _hptr(src), nbytes))


# ---- 1-bit Adam, compression stage -------------------------------------------------

def zero_onebit_state_init(dev_onebit, stream=None) -> None:
    _need("zero_onebit_state_init", dev_onebit, ONEBIT_STATE_BYTES)
    _check("zero_onebit_state_init", lib().zero_onebit_state_init(_ptr(dev_onebit), _stream(stream)))


def zero_onebit_workspace_bytes(n: int) -> int:
    return int(lib().zero_onebit_workspace_bytes(n))


def zero_onebit_step(p16, p32, m32, v32, err_w, err_s, grad16, n: int, bits_w, bits_s, dev_state, dev_onebit,
                     warmup: int, workspace, stream=None) -> None:
    for t, b in ((p16, 2), (p32, 4), (m32, 4), (v32, 4), (err_w, 4), (err_s, 4), (grad16, 2)):
        _need("zero_onebit_step", t, b * n)
    for t in (bits_w, bits_s):
        _need("zero_onebit_step", t, (n + 7) // 8)
    _need("zero_onebit_step", dev_state, STATE_BYTES)
    _need("zero_onebit_step", dev_onebit, ONEBIT_STATE_BYTES)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("zero_onebit_step",
           lib().zero_onebit_step(_ptr(p16), _ptr(p32), _ptr(m32), _ptr(v32), _ptr(err_w), _ptr(err_s),
                                  _ptr(grad16), n, _ptr(bits_w), _ptr(bits_s), _ptr(dev_state), _ptr(dev_onebit),
                                  int(warmup), _ptr(workspace), ws_bytes, _stream(stream)))


def read_onebit_state(dev_onebit) -> OneBitState:
    raw = dev_onebit.detach().to("cpu").numpy().tobytes()
    return OneBitState.from_buffer_copy(raw)
