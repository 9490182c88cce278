"""numpy-facing ctypes wrapper around the C oracle (liboracle_zero.so).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the benchmark's CPU-baseline leg import this module.  It imports nothing
from the HIP library or its binding.

The arithmetic lives in zero_oracle.c; this file only moves numpy arrays in
and out.  The per-function citations are in the C source.
"""
import ctypes as C

import numpy as np

from . import build as _build

_lib = None


class OracleSegment(C.Structure):
    _fields_ = [("src", C.c_void_p), ("src_off", C.c_uint64),
                ("dst_off", C.c_uint64), ("count", C.c_uint64)]


class OracleHParams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double),
                ("max_grad_norm", C.c_double), ("backoff", C.c_double),
                ("growth", C.c_double), ("min_scale", C.c_double),
                ("growth_interval", C.c_int32), ("reserved", C.c_int32)]


class OracleState(C.Structure):
    _fields_ = [("loss_scale", C.c_double), ("beta1_pow", C.c_double),
                ("beta2_pow", C.c_double), ("step", C.c_int64),
                ("good_steps", C.c_int32), ("skipped_total", C.c_int32),
                ("sumsq", C.c_double), ("grad_norm", C.c_double),
                ("overflow", C.c_int32), ("skip", C.c_int32),
                ("gmul", C.c_float), ("bc1", C.c_float), ("bc2", C.c_float),
                ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
                ("omb1", C.c_float), ("omb2", C.c_float), ("eps", C.c_float),
                ("wd", C.c_float)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(_build.ensure_built())
        vp, u64, u32, i32 = C.c_void_p, C.c_uint64, C.c_uint32, C.c_int32
        L.oracle_f32_from_f16.argtypes = [C.c_uint16]
        L.oracle_f32_from_f16.restype = C.c_float
        L.oracle_f16_from_f32.argtypes = [C.c_float]
        L.oracle_f16_from_f32.restype = C.c_uint16
        L.oracle_f16_from_f32_array.argtypes = [vp, vp, u64]
        L.oracle_f32_from_f16_array.argtypes = [vp, vp, u64]
        L.oracle_state_bytes.argtypes = [u64, u32, u32, C.c_int, C.POINTER(u64)]
        L.oracle_state_bytes.restype = C.c_int
        L.oracle_flatten.argtypes = [C.POINTER(OracleSegment), u32, vp, C.c_int, C.c_int]
        L.oracle_norm_overflow.argtypes = [vp, u64, C.POINTER(C.c_double), C.POINTER(i32)]
        L.oracle_norm_overflow_f32.argtypes = [vp, u64, C.POINTER(C.c_double), C.POINTER(i32)]
        L.oracle_adam_update_f32.argtypes = [C.POINTER(OracleState), vp, vp, vp, vp, vp, u64]
        L.oracle_onebit_scale.argtypes = [vp, u64, C.POINTER(C.c_double)]
        L.oracle_onebit_scale.restype = C.c_float
        L.oracle_onebit_pack.argtypes = [vp, u64, vp]
        L.oracle_onebit_step.argtypes = [C.POINTER(OracleState), vp, vp, vp, vp, vp, vp, vp, u64, vp, vp, vp]
        L.oracle_onebit_step.restype = C.c_int
        L.oracle_state_init.argtypes = [C.POINTER(OracleState), C.c_double]
        L.oracle_decide.argtypes = [C.POINTER(OracleState), C.POINTER(OracleHParams),
                                    C.c_double, i32]
        L.oracle_adam_update.argtypes = [C.POINTER(OracleState), vp, vp, vp, vp, vp, u64]
        L.oracle_step.argtypes = [C.POINTER(OracleHParams), C.POINTER(OracleState),
                                  C.POINTER(OracleSegment), u32, vp, vp, vp, vp, vp, u64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray, dtype) -> int:
    assert a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    return a.ctypes.data


# ---- binary16 conversions -------------------------------------------------

def f16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 array -> binary16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f16_from_f32_array(_ptr(x, np.float32), _ptr(out, np.uint16), x.size)
    return out


def f32_from_f16(h: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> exact fp32 values."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f32_from_f16_array(_ptr(h, np.uint16), _ptr(out, np.float32), h.size)
    return out


# ---- model-state bytes ------------------------------------------------------

def state_bytes(psi: int, nd: int, k: int = 12, stage: int = 3) -> int:
    out = C.c_uint64()
    rc = lib().oracle_state_bytes(psi, nd, k, stage, C.byref(out))
    if rc != 0:
        raise ValueError(f"oracle_state_bytes({psi}, {nd}, {k}, {stage}) rejected")
    return out.value


# ---- flatten ------------------------------------------------------------------

def flatten(srcs, segments, dst: np.ndarray, accumulate: bool = False) -> None:
    """segments: iterable of (tensor_index, src_off, dst_off, count) into srcs."""
    arr = (OracleSegment * max(1, len(segments)))()
    for j, (t, so, do, cnt) in enumerate(segments):
        arr[j] = OracleSegment(_ptr(srcs[t], np.uint16), so, do, cnt)
    if dst.dtype == np.float32:
        is32 = 1
    elif dst.dtype == np.uint16:
        is32 = 0
    else:
        raise TypeError(dst.dtype)
    assert dst.flags.c_contiguous
    lib().oracle_flatten(arr, len(segments), dst.ctypes.data, is32, int(bool(accumulate)))


# ---- norm / overflow ----------------------------------------------------------

def norm_overflow(g16: np.ndarray):
    """-> (sumsq: float, overflow: int) of a flat binary16 (uint16) array."""
    g16 = np.ascontiguousarray(g16, dtype=np.uint16)
    s = C.c_double()
    o = C.c_int32()
    lib().oracle_norm_overflow(_ptr(g16, np.uint16), g16.size, C.byref(s), C.byref(o))
    return s.value, o.value


def norm_overflow_f32(g32: np.ndarray):
    """-> (sumsq, overflow) of a flat fp32 gradient: overflow = some element is
    inf or NaN; sumsq = the exact sum of the exact squares, rounded once to
    binary64 (any finite values)."""
    g32 = np.ascontiguousarray(g32, dtype=np.float32)
    s = C.c_double()
    o = C.c_int32()
    lib().oracle_norm_overflow_f32(_ptr(g32, np.float32), g32.size, C.byref(s), C.byref(o))
    return s.value, o.value


# ---- decision + update ----------------------------------------------------------

def hparams(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
            max_grad_norm=1.0, backoff=0.5, growth=2.0, min_scale=1.0,
            growth_interval=20) -> OracleHParams:
    return OracleHParams(lr, beta1, beta2, eps, weight_decay, max_grad_norm,
                         backoff, growth, min_scale, growth_interval, 0)


def new_state(initial_scale: float) -> OracleState:
    st = OracleState()
    lib().oracle_state_init(C.byref(st), initial_scale)
    return st


def decide(st: OracleState, hp: OracleHParams, sumsq: float, overflow: int) -> None:
    lib().oracle_decide(C.byref(st), C.byref(hp), sumsq, int(overflow))


def adam_update(st: OracleState, p16, p32, m32, v32, g16) -> None:
    n = p32.size
    assert p16.size == m32.size == v32.size == g16.size == n
    lib().oracle_adam_update(C.byref(st), _ptr(p16, np.uint16), _ptr(p32, np.float32),
                             _ptr(m32, np.float32), _ptr(v32, np.float32),
                             _ptr(g16, np.uint16), n)


def adam_update_f32(st: OracleState, p16, p32, m32, v32, g32) -> None:
    n = p32.size
    assert p16.size == m32.size == v32.size == g32.size == n
    lib().oracle_adam_update_f32(C.byref(st), _ptr(p16, np.uint16), _ptr(p32, np.float32),
                                 _ptr(m32, np.float32), _ptr(v32, np.float32), _ptr(g32, np.float32), n)


def step(hp: OracleHParams, st: OracleState, srcs, segments, grad16, p16, p32, m32, v32) -> None:
    """One whole step: flatten, reduce, decide, update (all in C, one thread)."""
    arr = (OracleSegment * max(1, len(segments)))()
    for j, (t, so, do, cnt) in enumerate(segments):
        arr[j] = OracleSegment(_ptr(srcs[t], np.uint16), so, do, cnt)
    lib().oracle_step(C.byref(hp), C.byref(st), arr, len(segments), _ptr(grad16, np.uint16),
                      _ptr(p16, np.uint16), _ptr(p32, np.float32), _ptr(m32, np.float32),
                      _ptr(v32, np.float32), p32.size)


# ---- 1-bit Adam, compression stage -----------------------------------------------

def onebit_scale(x: np.ndarray):
    """-> (s, S): the fp32 scale ||x||_2/sqrt(d) from the exact sum of squares S."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    S = C.c_double()
    s = lib().oracle_onebit_scale(_ptr(x, np.float32), x.size, C.byref(S))
    return float(np.float32(s)), S.value


def onebit_pack(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros((x.size + 7) // 8, np.uint8)
    lib().oracle_onebit_pack(_ptr(x, np.float32), x.size, out.ctypes.data)
    return out


def onebit_step(st: OracleState, p16, p32, m32, v32, err_w, err_s, g16):
    """One compression-stage step; -> (bits_w, bits_s, (s_w, s_s))."""
    n = p32.size
    assert p16.size == m32.size == v32.size == err_w.size == err_s.size == g16.size == n
    bw = np.zeros((n + 7) // 8, np.uint8)
    bs = np.zeros((n + 7) // 8, np.uint8)
    sc = np.zeros(2, np.float32)
    rc = lib().oracle_onebit_step(C.byref(st), _ptr(p16, np.uint16), _ptr(p32, np.float32), _ptr(m32, np.float32),
                                  _ptr(v32, np.float32), _ptr(err_w, np.float32), _ptr(err_s, np.float32),
                                  _ptr(g16, np.uint16), n, bw.ctypes.data, bs.ctypes.data, sc.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_onebit_step")
    return bw, bs, (float(sc[0]), float(sc[1]))
