"""Python access to the plain CPU oracle (liboracle.so, float64 C loops).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.

The wrappers only marshal NumPy arrays into the C functions declared in
oracle.h; every step of the arithmetic is in oracle.c.  Storage conventions:
bf16 tensors are uint16 bit arrays, fp32 tensors are float32 arrays.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None

F32, BF16, F64 = 0, 1, 2

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        L.oracle_threads.restype = C.c_int
        L.oracle_threads.argtypes = []
        L.oracle_capacity.restype = _i32
        L.oracle_capacity.argtypes = [_i32, _i32, _i32, C.c_double]
        L.oracle_gate.restype = None
        L.oracle_gate.argtypes = [_i64, _i64, _i64, C.c_int, _p, _p, _p]
        L.oracle_route.restype = None
        L.oracle_route.argtypes = [_i64, _i64, _i64, _p, _p, C.c_int, C.c_int, _p, _p, _p]
        L.oracle_fp8_decode.restype = C.c_double
        L.oracle_fp8_decode.argtypes = [C.c_uint8]
        L.oracle_fp8_encode.restype = C.c_uint8
        L.oracle_fp8_encode.argtypes = [C.c_float]
        L.oracle_quantize_fp8.restype = None
        L.oracle_quantize_fp8.argtypes = [_i64, _i64, C.c_int, _p, _p, _p]
        L.oracle_dequantize_fp8.restype = None
        L.oracle_dequantize_fp8.argtypes = [_i64, _i64, _p, _p, _p]
        L.oracle_fp4_decode.restype = C.c_double
        L.oracle_fp4_decode.argtypes = [C.c_uint8]
        L.oracle_fp4_encode.restype = C.c_uint8
        L.oracle_fp4_encode.argtypes = [C.c_float]
        L.oracle_quantize_mxfp4.restype = None
        L.oracle_quantize_mxfp4.argtypes = [_i64, _i64, C.c_int, _p, _p, _p]
        L.oracle_dequantize_mxfp4.restype = None
        L.oracle_dequantize_mxfp4.argtypes = [_i64, _i64, _p, _p, _p]
        L.oracle_quantize_mxfp8.restype = None
        L.oracle_quantize_mxfp8.argtypes = [_i64, _i64, C.c_int, _p, _p, _p]
        L.oracle_dequantize_mxfp8.restype = None
        L.oracle_dequantize_mxfp8.argtypes = [_i64, _i64, _p, _p, _p]
        L.oracle_expert_ffn_a8.restype = None
        L.oracle_expert_ffn_a8.argtypes = [_i64, _i64, _i64, C.c_int, _p, C.c_int, _p, _p, _p, _p]
        L.oracle_load_stats.restype = None
        L.oracle_load_stats.argtypes = [_i64, _i64, _i64, _i32, _p, _p, _p, _p, _p]
        L.oracle_permute.restype = _i64
        L.oracle_permute.argtypes = [_i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _p]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [_i64, _i64, _i64, C.c_int, _p, C.c_int, _p, _p, _p, _p]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.oracle_layer.restype = _i64
        L.oracle_layer.argtypes = [_i64] * 6 + [_i32, C.c_int, C.c_int, C.c_int] + [_p] * 15
        _lib = L
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs are bf16 bits (uint16), float32 or float64, got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def threads() -> int:
    return int(lib().oracle_threads())


def capacity(T: int, k: int, E: int, factor: float | None) -> int:
    """-1 (unlimited) when factor is None."""
    if factor is None:
        return -1
    return int(lib().oracle_capacity(T, k, E, factor))


def gate(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    x, wg = _c(x), _c(wg)
    assert _dt(x) == _dt(wg)
    T, H = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), np.float32)
    lib().oracle_gate(T, H, E, _dt(x), _ptr(x), _ptr(wg), _ptr(out))
    return out


BIAS_SOFTMAX, BIAS_SELECT = 0, 1


def route(logits: np.ndarray, k: int, bias: np.ndarray | None = None, renormalize: int = 1,
          bias_mode: int = BIAS_SOFTMAX):
    """Returns (ids int32 [T,k], w float64 [T,k], margin float64 [T])."""
    logits = _c(logits, np.float32)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    margin = np.empty((T,), np.float64)
    lib().oracle_route(T, E, k, _ptr(logits), _ptr(bias), int(renormalize), int(bias_mode),
                       _ptr(ids), _ptr(w), _ptr(margin))
    return ids, w, margin


def load_stats(ids: np.ndarray, E: int, capacity: int = -1, bias_next: bool = False):
    """Per-expert picks and the load statistics of a routing decision (oracle_load_stats);
    with bias_next, also the next balancing bias (float32 [E], needs capacity >= 1)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    raw = np.empty(E, np.int32)
    ints = np.empty(6, np.int64)
    reals = np.empty(5, np.float64)
    b = np.empty(E, np.float32) if bias_next else None
    lib().oracle_load_stats(T, E, k, int(capacity), _ptr(ids), _ptr(raw), _ptr(ints), _ptr(reals),
                            _ptr(b))
    out = dict(raw=raw, picks=int(ints[0]), dropped=int(ints[1]), max_count=int(ints[2]),
               hottest=int(ints[3]), min_count=int(ints[4]), idle=int(ints[5]),
               mean=float(reals[0]), stddev=float(reals[1]), cv=float(reals[2]),
               max_over_mean=float(reals[3]), drop_rate=float(reals[4]))
    if bias_next:
        out["bias_next"] = b
    return out


def permute(ids: np.ndarray, E: int, capacity: int = -1, active: np.ndarray | None = None):
    """Returns a dict with raw, counts, offsets, row_token, pos, dropped, n_dropped."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    if active is not None:
        active = _c(active, np.uint8)
    raw = np.empty(E, np.int32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_token = np.full(max(T * k, 1), -1, np.int32)
    pos = np.empty((T, k), np.int32)
    dropped = np.empty((T, k), np.uint8)
    nd = lib().oracle_permute(T, E, k, int(capacity), _ptr(ids), _ptr(active), _ptr(raw),
                              _ptr(counts), _ptr(offsets), _ptr(row_token), _ptr(pos),
                              _ptr(dropped))
    R = int(offsets[E])
    return dict(raw=raw, counts=counts, offsets=offsets, row_token=row_token[:R], pos=pos,
                dropped=dropped, n_dropped=int(nd))


def fp8_decode(code: int) -> float:
    return float(lib().oracle_fp8_decode(int(code)))


def fp8_encode(x: float) -> int:
    return int(lib().oracle_fp8_encode(float(x)))


def quantize_fp8(w: np.ndarray):
    """Per-row FP8 E4M3 quantisation of a [rows, K] bf16-bits or float32 matrix (any leading
    shape is flattened into rows).  Returns (codes uint8, same shape; scales float32 [rows])."""
    w = _c(w)
    K = w.shape[-1]
    rows = w.size // K if K else 0
    q = np.empty(w.shape, np.uint8)
    sc = np.empty(w.shape[:-1], np.float32)
    lib().oracle_quantize_fp8(rows, K, _dt(w), _ptr(w), _ptr(q), _ptr(sc))
    return q, sc


def dequantize_fp8(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.float32)
    K = q.shape[-1]
    out = np.empty(q.shape, np.float64)
    lib().oracle_dequantize_fp8(q.size // K if K else 0, K, _ptr(q), _ptr(scales), _ptr(out))
    return out


def fp4_decode(code: int) -> float:
    return float(lib().oracle_fp4_decode(int(code)))


def fp4_encode(x: float) -> int:
    return int(lib().oracle_fp4_encode(float(x)))


def quantize_mxfp4(w: np.ndarray):
    """MXFP4 quantisation of a [..., K] bf16-bits or float32 matrix (K % 32 == 0).  Returns
    (codes uint8 [..., K/2], two per byte, low nibble first; scales uint8 [..., K/32], E8M0)."""
    w = _c(w)
    K = w.shape[-1]
    rows = w.size // K if K else 0
    q = np.empty(w.shape[:-1] + (K // 2,), np.uint8)
    sc = np.empty(w.shape[:-1] + (K // 32,), np.uint8)
    lib().oracle_quantize_mxfp4(rows, K, _dt(w), _ptr(w), _ptr(q), _ptr(sc))
    return q, sc


def dequantize_mxfp4(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.uint8)
    K = q.shape[-1] * 2
    out = np.empty(q.shape[:-1] + (K,), np.float64)
    lib().oracle_dequantize_mxfp4(q.size * 2 // K if K else 0, K, _ptr(q), _ptr(scales), _ptr(out))
    return out


def quantize_mxfp8(x: np.ndarray):
    """MXFP8 quantisation of a [..., K] bf16-bits, float32 or float64 matrix (K % 32 == 0).
    Returns (codes uint8 [..., K], E4M3; scales uint8 [..., K/32], E8M0)."""
    x = _c(x)
    K = x.shape[-1]
    rows = x.size // K if K else 0
    q = np.empty(x.shape, np.uint8)
    sc = np.empty(x.shape[:-1] + (K // 32,), np.uint8)
    lib().oracle_quantize_mxfp8(rows, K, _dt(x), _ptr(x), _ptr(q), _ptr(sc))
    return q, sc


def dequantize_mxfp8(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    q = _c(q, np.uint8)
    scales = _c(scales, np.uint8)
    K = q.shape[-1]
    out = np.empty(q.shape, np.float64)
    lib().oracle_dequantize_mxfp8(q.size // K if K else 0, K, _ptr(q), _ptr(scales), _ptr(out))
    return out


def expert_ffn_a8(xr: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """The SwiGLU FFN with MXFP8 activations (input rows and the gate-up output quantised)."""
    xr, w1, w3, w2 = _c(xr), _c(w1), _c(w3), _c(w2)
    M, H = xr.shape
    I = w1.shape[0]
    assert w1.shape == (I, H) and w3.shape == (I, H) and w2.shape == (H, I)
    assert _dt(w1) == _dt(w3) == _dt(w2) and H % 32 == 0 and I % 32 == 0
    out = np.empty((M, H), np.float64)
    if M:
        lib().oracle_expert_ffn_a8(M, H, I, _dt(xr), _ptr(xr), _dt(w1), _ptr(w1), _ptr(w3),
                                   _ptr(w2), _ptr(out))
    return out


def expert_ffn(xr: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    xr, w1, w3, w2 = _c(xr), _c(w1), _c(w3), _c(w2)
    M, H = xr.shape
    I = w1.shape[0]
    assert w1.shape == (I, H) and w3.shape == (I, H) and w2.shape == (H, I)
    assert _dt(w1) == _dt(w3) == _dt(w2)
    out = np.empty((M, H), np.float64)
    if M:
        lib().oracle_expert_ffn(M, H, I, _dt(xr), _ptr(xr), _dt(w1), _ptr(w1), _ptr(w3), _ptr(w2),
                                _ptr(out))
    return out


def combine(yp: np.ndarray, pos: np.ndarray, w: np.ndarray, ys: np.ndarray | None = None):
    yp = _c(yp, np.float64)
    pos = _c(pos, np.int32)
    w = _c(w, np.float64)
    ys = _c(ys, np.float64)
    T, k = pos.shape
    H = yp.shape[1] if yp.ndim == 2 and yp.shape[0] else (ys.shape[1] if ys is not None else 0)
    if yp.ndim != 2 or yp.shape[0] == 0:
        yp = np.zeros((1, H), np.float64)
    y = np.empty((T, H), np.float64)
    lib().oracle_combine(T, H, k, _ptr(yp), _ptr(pos), _ptr(w), _ptr(ys), _ptr(y))
    return y


def layer(x, wg, w1, w3, w2, k, capacity=-1, renormalize=1, bias=None, shared=None,
          bias_mode=BIAS_SOFTMAX):
    """Whole layer; returns (y float64 [T,H], info dict)."""
    x, wg, w1, w3, w2 = _c(x), _c(wg), _c(w1), _c(w3), _c(w2)
    bias = _c(bias, np.float32)
    dt = _dt(x)
    T, H = x.shape
    E, I = w1.shape[0], w1.shape[1]
    if shared is not None:
        ws1, ws3, ws2 = (_c(a) for a in shared)
        Is = ws1.shape[0]
    else:
        ws1 = ws3 = ws2 = None
        Is = 0
    y = np.empty((T, H), np.float64)
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    pos = np.empty((T, k), np.int32)
    counts = np.empty(E, np.int32)
    nd = lib().oracle_layer(T, H, E, k, I, Is, int(capacity), int(renormalize), int(bias_mode),
                            dt, _ptr(x),
                            _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(ws1),
                            _ptr(ws3), _ptr(ws2), _ptr(y), _ptr(logits), _ptr(ids), _ptr(w),
                            _ptr(pos), _ptr(counts))
    return y, dict(logits=logits, ids=ids, w=w, pos=pos, counts=counts, n_dropped=int(nd))
