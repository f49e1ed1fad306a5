"""Thin torch-tensor binding of libmoe.so.

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed along, status codes become exceptions.  Every step of the
layer runs in the library's HIP kernels.  PyTorch provides device memory and
streams.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MoeCacheStep, MoeDebugOut, MoeDims, MoeError, MoeLoadStats

_DT = {"bf16": _lib.MOE_BF16, "f32": _lib.MOE_F32}
_BIAS = {"softmax": _lib.MOE_BIAS_SOFTMAX, "select": _lib.MOE_BIAS_SELECT}
_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass(frozen=True)
class Dims:
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int = 0
    capacity: int = -1
    renormalize: int = 1
    dtype: str = "bf16"
    bias_mode: str = "softmax"  # "softmax": bias inside the softmax; "select": ranking only

    def c(self) -> MoeDims:
        return MoeDims(self.T, self.H, self.E, self.k, self.I, self.I_shared, self.capacity,
                       self.renormalize, _DT[self.dtype], _BIAS[self.bias_mode])

    @property
    def torch_dtype(self):
        return _TORCH_DT[self.dtype]


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status, where):
    if status != _lib.MOE_OK:
        raise MoeError(status, where)


def capacity(T: int, k: int, E: int, factor: float) -> int:
    return int(_lib.lib().moe_capacity(T, k, E, factor))


def workspace_bytes(d: Dims) -> int:
    c = d.c()
    return int(_lib.lib().moe_workspace_bytes(C.byref(c)))


def workspace(d: Dims, device="cuda") -> torch.Tensor:
    n = workspace_bytes(d)
    if n == 0:
        raise ValueError(f"invalid dims {d}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def gate(d: Dims, x, wg, logits, stream=None):
    c = d.c()
    _check(_lib.lib().moe_gate(C.byref(c), _ptr(x, d.torch_dtype, "x"),
                               _ptr(wg, d.torch_dtype, "wg"),
                               _ptr(logits, torch.float32, "logits"), _stream(stream)), "moe_gate")


def route(d: Dims, logits, bias, ids, w, counts=None, dropped=None, n_dropped=None, ws=None,
          stream=None):
    c = d.c()
    _check(_lib.lib().moe_route(
        C.byref(c), _ptr(logits, torch.float32, "logits"), _ptr(bias, torch.float32, "bias"),
        _ptr(ids, torch.int32, "ids"), _ptr(w, torch.float32, "w"),
        _ptr(counts, torch.int32, "counts"), _ptr(dropped, torch.uint8, "dropped"),
        _ptr(n_dropped, torch.int32, "n_dropped"), _ptr(ws, torch.uint8, "ws"),
        0 if ws is None else ws.numel(), _stream(stream)), "moe_route")


def permute(d: Dims, x, ids, dropped, offsets, row_token, pos, x_packed, ws, stream=None):
    c = d.c()
    _check(_lib.lib().moe_permute(
        C.byref(c), _ptr(x, d.torch_dtype, "x"), _ptr(ids, torch.int32, "ids"),
        _ptr(dropped, torch.uint8, "dropped"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(row_token, torch.int32, "row_token"), _ptr(pos, torch.int32, "pos"),
        _ptr(x_packed, d.torch_dtype, "x_packed"), _ptr(ws, torch.uint8, "ws"),
        0 if ws is None else ws.numel(), _stream(stream)), "moe_permute")


def expert_ffn(d: Dims, x_packed, offsets, w1, w3, w2, y_packed, ws, stream=None):
    c = d.c()
    dt = d.torch_dtype
    _check(_lib.lib().moe_expert_ffn(
        C.byref(c), _ptr(x_packed, dt, "x_packed"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(w1, dt, "w1"), _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(y_packed, dt, "y_packed"),
        _ptr(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)),
        "moe_expert_ffn")


def combine(d: Dims, y_packed, pos, w, y_shared, y, stream=None):
    c = d.c()
    dt = d.torch_dtype
    _check(_lib.lib().moe_combine(
        C.byref(c), _ptr(y_packed, dt, "y_packed"), _ptr(pos, torch.int32, "pos"),
        _ptr(w, torch.float32, "w"), _ptr(y_shared, dt, "y_shared"), _ptr(y, dt, "y"),
        _stream(stream)), "moe_combine")


# fields of moe_load_stats_t, in order
LOAD_STATS_FIELDS = tuple(f for f, _ in MoeLoadStats._fields_)


def load_stats_buffer(device="cuda") -> torch.Tensor:
    """Device bytes for one moe_load_stats_t."""
    return torch.zeros(C.sizeof(MoeLoadStats), dtype=torch.uint8, device=device)


def read_load_stats(buf: torch.Tensor) -> dict:
    """Host copy of a moe_load_stats_t written by load_stats (synchronises)."""
    raw = bytes(buf.cpu().numpy().tobytes())
    s = MoeLoadStats.from_buffer_copy(raw)
    return {f: getattr(s, f) for f in LOAD_STATS_FIELDS}


def load_stats(d: Dims, ids, stats, raw_counts=None, bias_next=None, ws=None, stream=None):
    """Per-expert picks, load statistics into `stats` (load_stats_buffer) and, optionally, the
    next balancing bias."""
    c = d.c()
    _check(_lib.lib().moe_load_stats(
        C.byref(c), _ptr(ids, torch.int32, "ids"), _ptr(raw_counts, torch.int32, "raw_counts"),
        _ptr(stats, torch.uint8, "stats"), _ptr(bias_next, torch.float32, "bias_next"),
        _ptr(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)),
        "moe_load_stats")


def quantize_fp8(w, q=None, scales=None, stream=None):
    """Per-row FP8 E4M3 quantisation of a bf16 or fp32 device tensor (rows = all leading
    dimensions).  Returns (codes uint8 of w's shape, scales float32 of w's leading shape)."""
    dt = {torch.bfloat16: _lib.MOE_BF16, torch.float32: _lib.MOE_F32}.get(w.dtype)
    if dt is None:
        raise TypeError(f"quantize_fp8: bf16 or fp32 weights, got {w.dtype}")
    K = w.shape[-1]
    rows = w.numel() // K
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    _check(_lib.lib().moe_quantize_fp8(rows, K, dt, _ptr(w, None, "w"), _ptr(q, torch.uint8, "q"),
                                       _ptr(scales, torch.float32, "scales"), _stream(stream)),
           "moe_quantize_fp8")
    return q, scales


def quantize_mxfp4(w, q=None, scales=None, stream=None):
    """MXFP4 quantisation of a bf16 or fp32 device tensor [..., R, K] (R % 32 == 0,
    K % 128 == 0).  Returns (E2M1 codes uint8 [..., R/32, K/128, 32 * 64], two per byte, low
    nibble first: [r/32, k/128, (r%32)*64 + (k%128)/2] holds element k of row r; E8M0 scales
    uint8 [..., R/32, K/128, 32 * 4]: [r/32, b/4, (r%32)*4 + b%4] holds the scale of row r,
    32-block b) -- both blocked by 32 rows and 128 k."""
    dt = {torch.bfloat16: _lib.MOE_BF16, torch.float32: _lib.MOE_F32}.get(w.dtype)
    if dt is None:
        raise TypeError(f"quantize_mxfp4: bf16 or fp32 weights, got {w.dtype}")
    if w.dim() < 2:
        raise ValueError("quantize_mxfp4: weights [..., R, K]")
    R, K = w.shape[-2], w.shape[-1]
    rows = w.numel() // K
    if q is None:
        q = torch.empty(w.shape[:-2] + (R // 32, K // 128, 2048), dtype=torch.uint8,
                        device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-2] + (R // 32, K // 128, 128), dtype=torch.uint8,
                             device=w.device)
    _check(_lib.lib().moe_quantize_mxfp4(rows, K, dt, _ptr(w, None, "w"), _ptr(q, torch.uint8, "q"),
                                         _ptr(scales, torch.uint8, "scales"), _stream(stream)),
           "moe_quantize_mxfp4")
    return q, scales


def quantize_mxfp8(x, q=None, scales=None, stream=None):
    """MXFP8 quantisation of a bf16 or fp32 device tensor [..., K] (K % 32 == 0).  Returns
    (E4M3 codes uint8 of x's shape, E8M0 scales uint8 [..., K/32]), both row-major."""
    dt = {torch.bfloat16: _lib.MOE_BF16, torch.float32: _lib.MOE_F32}.get(x.dtype)
    if dt is None:
        raise TypeError(f"quantize_mxfp8: bf16 or fp32 input, got {x.dtype}")
    K = x.shape[-1]
    rows = x.numel() // K if K else 0
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (K // 32,), dtype=torch.uint8, device=x.device)
    _check(_lib.lib().moe_quantize_mxfp8(rows, K, dt, _ptr(x, None, "x"), _ptr(q, torch.uint8, "q"),
                                         _ptr(scales, torch.uint8, "scales"), _stream(stream)),
           "moe_quantize_mxfp8")
    return q, scales


def expert_ffn_mxfp4(d: Dims, x_packed, offsets, w1, w3, w2, y_packed, ws, stream=None,
                     _entry="moe_expert_ffn_mxfp4"):
    """moe_expert_ffn_mxfp4; w1, w3, w2 are (codes, scales) pairs from quantize_mxfp4."""
    c = d.c()
    dt = d.torch_dtype
    (q1, s1), (q3, s3), (q2, s2) = w1, w3, w2
    u8 = torch.uint8
    _check(getattr(_lib.lib(), _entry)(
        C.byref(c), _ptr(x_packed, dt, "x_packed"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(q1, u8, "w1q"), _ptr(s1, u8, "w1s"), _ptr(q3, u8, "w3q"), _ptr(s3, u8, "w3s"),
        _ptr(q2, u8, "w2q"), _ptr(s2, u8, "w2s"), _ptr(y_packed, dt, "y_packed"),
        _ptr(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)),
        _entry)


def expert_ffn_w4a8(d: Dims, x_packed, offsets, w1, w3, w2, y_packed, ws, stream=None):
    """moe_expert_ffn_w4a8: MXFP4 weights ((codes, scales) pairs from quantize_mxfp4) on
    MXFP8 activations (x_packed is bf16; the call quantises it)."""
    expert_ffn_mxfp4(d, x_packed, offsets, w1, w3, w2, y_packed, ws, stream,
                     _entry="moe_expert_ffn_w4a8")


def layer_forward_w4a8(d: Dims, x, wg, bias, w1, w3, w2, shared=None, y=None, ws=None,
                       debug=None, stream=None):
    """The fused layer with MXFP4 expert weights on MXFP8 activations (arguments as
    layer_forward_mxfp4).  Returns y."""
    return layer_forward_mxfp4(d, x, wg, bias, w1, w3, w2, shared, y, ws, debug, stream,
                               _entry="moe_layer_forward_w4a8")


def layer_forward_mxfp4(d: Dims, x, wg, bias, w1, w3, w2, shared=None, y=None, ws=None,
                        debug=None, stream=None, _entry="moe_layer_forward_mxfp4"):
    """The fused layer with MXFP4 expert weights ((codes, scales) pairs from quantize_mxfp4,
    the shared expert's in `shared`).  Returns y."""
    dt = d.torch_dtype
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(d, x.device)
    u8 = torch.uint8
    none = (None, None)
    (q1, s1), (q3, s3), (q2, s2) = w1, w3, w2
    (e1, t1), (e3, t3), (e2, t2) = shared if shared is not None else (none, none, none)
    dbg = _debug_struct(debug) if debug else None
    c = d.c()
    _check(getattr(_lib.lib(), _entry)(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, torch.float32, "bias"),
        _ptr(q1, u8, "w1q"), _ptr(s1, u8, "w1s"), _ptr(q3, u8, "w3q"), _ptr(s3, u8, "w3s"),
        _ptr(q2, u8, "w2q"), _ptr(s2, u8, "w2s"), _ptr(e1, u8, "ws1q"), _ptr(t1, u8, "ws1s"),
        _ptr(e3, u8, "ws3q"), _ptr(t3, u8, "ws3s"), _ptr(e2, u8, "ws2q"), _ptr(t2, u8, "ws2s"),
        _ptr(y, dt, "y"), C.byref(dbg) if dbg is not None else None, _ptr(ws, torch.uint8, "ws"),
        ws.numel(), _stream(stream)), _entry)
    return y


def expert_ffn_fp8(d: Dims, x_packed, offsets, w1, w3, w2, y_packed, ws, stream=None):
    """moe_expert_ffn_fp8; w1, w3, w2 are (codes, scales) pairs from quantize_fp8."""
    c = d.c()
    dt = d.torch_dtype
    (q1, s1), (q3, s3), (q2, s2) = w1, w3, w2
    u8, f32 = torch.uint8, torch.float32
    _check(_lib.lib().moe_expert_ffn_fp8(
        C.byref(c), _ptr(x_packed, dt, "x_packed"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(q1, u8, "w1q"), _ptr(s1, f32, "w1s"), _ptr(q3, u8, "w3q"), _ptr(s3, f32, "w3s"),
        _ptr(q2, u8, "w2q"), _ptr(s2, f32, "w2s"), _ptr(y_packed, dt, "y_packed"),
        _ptr(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)),
        "moe_expert_ffn_fp8")


def _debug_struct(debug):
    types = dict(logits=torch.float32, topk_ids=torch.int32, topk_w=torch.float32,
                 counts=torch.int32, offsets=torch.int32, pos=torch.int32, n_dropped=torch.int32)
    dbg = MoeDebugOut(**{k: _ptr(v, types[k], k) for k, v in debug.items() if k != "events"})
    for i, ev in enumerate(debug.get("events") or []):
        dbg.events[i] = ev  # raw hipEvent_t handles (or None)
    return dbg


def layer_forward_fp8(d: Dims, x, wg, bias, w1, w3, w2, shared=None, y=None, ws=None,
                      debug=None, stream=None):
    """The fused layer with FP8 expert weights: w1, w3, w2 (and the three shared-expert weights
    in `shared`) are (codes, scales) pairs from quantize_fp8.  Returns y."""
    dt = d.torch_dtype
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(d, x.device)
    u8, f32 = torch.uint8, torch.float32
    none = (None, None)
    (q1, s1), (q3, s3), (q2, s2) = w1, w3, w2
    (e1, t1), (e3, t3), (e2, t2) = shared if shared is not None else (none, none, none)
    dbg = _debug_struct(debug) if debug else None
    c = d.c()
    _check(_lib.lib().moe_layer_forward_fp8(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, f32, "bias"),
        _ptr(q1, u8, "w1q"), _ptr(s1, f32, "w1s"), _ptr(q3, u8, "w3q"), _ptr(s3, f32, "w3s"),
        _ptr(q2, u8, "w2q"), _ptr(s2, f32, "w2s"), _ptr(e1, u8, "ws1q"), _ptr(t1, f32, "ws1s"),
        _ptr(e3, u8, "ws3q"), _ptr(t3, f32, "ws3s"), _ptr(e2, u8, "ws2q"), _ptr(t2, f32, "ws2s"),
        _ptr(y, dt, "y"), C.byref(dbg) if dbg is not None else None, _ptr(ws, torch.uint8, "ws"),
        ws.numel(), _stream(stream)), "moe_layer_forward_fp8")
    return y


def _step_dict(info: MoeCacheStep) -> dict:
    return {f: getattr(info, f) for f, _ in MoeCacheStep._fields_}


class ExpertCache:
    """An expert cache (moe_cache_*): `slots` experts of the routed weights resident in a device
    pool, the rest in host memory (w1, w3 [E, I, H] and w2 [E, H, I], bf16 CPU tensors; pin
    them for asynchronous copies).  The host tensors must outlive the cache."""

    def __init__(self, d: Dims, slots: int, w1, w3, w2, device="cuda"):
        """w1, w3, w2: bf16 host tensors, or (for an MXFP4 cache) (codes, scales) pairs of uint8
        host tensors as quantize_mxfp4 returns them for [E, I, H] and [E, H, I]."""
        self.mxfp4 = isinstance(w1, tuple)
        parts = [a for w in (w1, w3, w2) for a in (w if self.mxfp4 else (w,))]
        want = torch.uint8 if self.mxfp4 else d.torch_dtype
        for t in parts:
            if t.is_cuda or t.dtype != want or not t.is_contiguous():
                raise ValueError(f"expert weights: contiguous host tensors of {want} expected")
        self._keep = parts
        self.d = d
        c = d.c()
        L = _lib.lib()
        pool_bytes = L.moe_cache_pool_bytes_mxfp4 if self.mxfp4 else L.moe_cache_pool_bytes
        n = int(pool_bytes(C.byref(c), slots))
        if n == 0:
            raise ValueError(f"invalid cache dims {d} / slots {slots}")
        self.pool = torch.empty(n, dtype=torch.uint8, device=device)
        h = C.c_void_p()
        ptrs = [t.data_ptr() for t in parts]
        if self.mxfp4:
            _check(L.moe_cache_create_mxfp4(C.byref(c), slots, *ptrs, self.pool.data_ptr(), n,
                                            C.byref(h)), "moe_cache_create_mxfp4")
        else:
            _check(L.moe_cache_create(C.byref(c), slots, *ptrs, self.pool.data_ptr(), n,
                                      C.byref(h)), "moe_cache_create")
        self.handle = h

    def load(self, experts, copy_stream=None, stream=None, wait=True):
        """Make `experts` resident (a prefetch).  wait: also wait for the step and return its
        report (else return None at once)."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        info = MoeCacheStep()
        _check(_lib.lib().moe_cache_load(self.handle, ids.ctypes.data if ids.size else None,
                                         int(ids.size), _stream(copy_stream), _stream(stream),
                                         C.byref(info) if wait else None), "moe_cache_load")
        return _step_dict(info) if wait else None

    def last_step(self) -> dict:
        """The report of the cache's last residency step (waits for it)."""
        info = MoeCacheStep()
        _check(_lib.lib().moe_cache_last_step(self.handle, C.byref(info)), "moe_cache_last_step")
        return _step_dict(info)

    def slots(self):
        import numpy as np
        out = np.empty(self.d.E, np.int32)
        _check(_lib.lib().moe_cache_slots(self.handle, out.ctypes.data), "moe_cache_slots")
        return out

    def close(self):
        if getattr(self, "handle", None):
            _lib.lib().moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


def layer_forward_cached(d: Dims, x, wg, bias, cache: ExpertCache, shared=None, y=None, ws=None,
                         debug=None, stream=None, copy_stream=None, wait=True):
    """The fused layer with the routed experts' weights in an ExpertCache; returns (y, step
    info).  wait: wait for the layer's residency step at the end and report it (else the call
    only enqueues and the info is None; ExpertCache.last_step reports it later)."""
    dt = d.torch_dtype
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(d, x.device)
    s1 = s3 = s2 = None
    if shared is not None:
        s1, s3, s2 = shared
    dbg = _debug_struct(debug) if debug else None
    info = MoeCacheStep()
    c = d.c()
    _check(_lib.lib().moe_layer_forward_cached(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, torch.float32, "bias"),
        cache.handle, _ptr(s1, dt, "ws1"), _ptr(s3, dt, "ws3"), _ptr(s2, dt, "ws2"), _ptr(y, dt, "y"),
        C.byref(dbg) if dbg is not None else None, _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream), _stream(copy_stream if copy_stream is not None else stream),
        C.byref(info) if wait else None), "moe_layer_forward_cached")
    return y, (_step_dict(info) if wait else None)


def layer_forward_cached_w4a8(d: Dims, x, wg, bias, cache: ExpertCache, shared=None, y=None,
                              ws=None, debug=None, stream=None, copy_stream=None, wait=True):
    """The fused layer on MXFP8 activations with the routed experts' MXFP4 weights in an MXFP4
    ExpertCache; shared: the shared expert's (codes, scales) pairs on the device, or None.
    Returns (y, step info)."""
    dt = d.torch_dtype
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(d, x.device)
    none = (None, None)
    (e1, t1), (e3, t3), (e2, t2) = shared if shared is not None else (none, none, none)
    u8 = torch.uint8
    dbg = _debug_struct(debug) if debug else None
    info = MoeCacheStep()
    c = d.c()
    _check(_lib.lib().moe_layer_forward_cached_w4a8(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, torch.float32, "bias"),
        cache.handle, _ptr(e1, u8, "ws1q"), _ptr(t1, u8, "ws1s"), _ptr(e3, u8, "ws3q"),
        _ptr(t3, u8, "ws3s"), _ptr(e2, u8, "ws2q"), _ptr(t2, u8, "ws2s"), _ptr(y, dt, "y"),
        C.byref(dbg) if dbg is not None else None, _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream), _stream(copy_stream if copy_stream is not None else stream),
        C.byref(info) if wait else None), "moe_layer_forward_cached_w4a8")
    return y, (_step_dict(info) if wait else None)


def layer_forward(d: Dims, x, wg, bias, w1, w3, w2, shared=None, y=None, ws=None, debug=None,
                  stream=None):
    """The fused layer.  shared = (ws1, ws3, ws2) or None; debug: dict of tensors to fill
    (keys: logits, topk_ids, topk_w, counts, offsets, pos, n_dropped).  Returns y."""
    dt = d.torch_dtype
    if y is None:
        y = torch.empty((d.T, d.H), dtype=dt, device=x.device)
    if ws is None:
        ws = workspace(d, x.device)
    s1 = s3 = s2 = None
    if shared is not None:
        s1, s3, s2 = shared
    dbg = _debug_struct(debug) if debug else None
    c = d.c()
    _check(_lib.lib().moe_layer_forward(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, torch.float32, "bias"),
        _ptr(w1, dt, "w1"), _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(s1, dt, "ws1"),
        _ptr(s3, dt, "ws3"), _ptr(s2, dt, "ws2"), _ptr(y, dt, "y"),
        C.byref(dbg) if dbg is not None else None, _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_layer_forward")
    return y


def static_scratch_bytes() -> int:
    """Bytes of the library-owned scratch array moe_layer_forward_static uses (per device)."""
    return int(_lib.lib().moe_static_scratch_bytes())


def layer_forward_static(d: Dims, x, wg, bias, w1, w3, w2, y, shared=None, debug=None,
                         stream=None):
    """The fused layer on the library's own scratch array (no workspace, nothing allocated by
    the call).  y must be given: this entry point is for callers that cannot allocate."""
    dt = d.torch_dtype
    s1 = s3 = s2 = None
    if shared is not None:
        s1, s3, s2 = shared
    dbg = _debug_struct(debug) if debug else None
    c = d.c()
    _check(_lib.lib().moe_layer_forward_static(
        C.byref(c), _ptr(x, dt, "x"), _ptr(wg, dt, "wg"), _ptr(bias, torch.float32, "bias"),
        _ptr(w1, dt, "w1"), _ptr(w3, dt, "w3"), _ptr(w2, dt, "w2"), _ptr(s1, dt, "ws1"),
        _ptr(s3, dt, "ws3"), _ptr(s2, dt, "ws2"), _ptr(y, dt, "y"),
        C.byref(dbg) if dbg is not None else None, _stream(stream)), "moe_layer_forward_static")
    return y
