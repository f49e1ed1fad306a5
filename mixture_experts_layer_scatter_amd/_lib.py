"""ctypes declarations of libmoe.so (include/moe.h).  Loading fails loudly when
the library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

# every symbol include/moe.h declares
EXPORTS = ("moe_status_str", "moe_capacity", "moe_workspace_bytes", "moe_gate", "moe_route",
           "moe_permute", "moe_expert_ffn", "moe_combine", "moe_load_stats", "moe_quantize_fp8",
           "moe_expert_ffn_fp8", "moe_quantize_mxfp4", "moe_expert_ffn_mxfp4",
           "moe_layer_forward_mxfp4", "moe_cache_pool_bytes", "moe_cache_create", "moe_cache_destroy",
           "moe_cache_load", "moe_cache_slots", "moe_layer_forward", "moe_layer_forward_fp8",
           "moe_layer_forward_cached", "moe_static_scratch_bytes", "moe_layer_forward_static",
           "moe_quantize_mxfp8", "moe_expert_ffn_w4a8", "moe_layer_forward_w4a8",
           "moe_cache_pool_bytes_mxfp4", "moe_cache_create_mxfp4", "moe_layer_forward_cached_w4a8",
           "moe_cache_last_step")
MOE_BIAS_SOFTMAX, MOE_BIAS_SELECT = 0, 1


class MoeDims(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("I", C.c_int32), ("I_shared", C.c_int32), ("capacity", C.c_int32),
                ("renormalize", C.c_int32), ("dtype", C.c_int32), ("bias_mode", C.c_int32)]


class MoeLoadStats(C.Structure):
    _fields_ = [("picks", C.c_int32), ("dropped", C.c_int32), ("max_count", C.c_int32),
                ("hottest", C.c_int32), ("min_count", C.c_int32), ("idle", C.c_int32),
                ("mean", C.c_float), ("stddev", C.c_float), ("cv", C.c_float),
                ("max_over_mean", C.c_float), ("drop_rate", C.c_float)]


class MoeCacheStep(C.Structure):
    _fields_ = [("requested", C.c_int32), ("hits", C.c_int32), ("loads", C.c_int32),
                ("evictions", C.c_int32), ("bytes_loaded", C.c_int64)]


class MoeDebugOut(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("pos", C.c_void_p),
                ("n_dropped", C.c_void_p), ("events", C.c_void_p * 7)]

# stage boundaries of moe_layer_forward (MOE_EV_* in include/moe.h)
EV_START, EV_GATE, EV_ROUTE, EV_PERMUTE, EV_GATE_UP, EV_DOWN, EV_END, NUM_EVENTS = range(8)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc, gfx950) first")
        L = C.CDLL(LIB_PATH)
        p, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        D = C.POINTER(MoeDims)
        L.moe_status_str.restype = C.c_char_p
        L.moe_status_str.argtypes = [i32]
        L.moe_capacity.restype = i32
        L.moe_capacity.argtypes = [i32, i32, i32, C.c_double]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [D]
        L.moe_gate.restype = i32
        L.moe_gate.argtypes = [D, p, p, p, p]
        L.moe_route.restype = i32
        L.moe_route.argtypes = [D, p, p, p, p, p, p, p, p, sz, p]
        L.moe_permute.restype = i32
        L.moe_permute.argtypes = [D, p, p, p, p, p, p, p, p, sz, p]
        L.moe_expert_ffn.restype = i32
        L.moe_expert_ffn.argtypes = [D, p, p, p, p, p, p, p, sz, p]
        L.moe_combine.restype = i32
        L.moe_combine.argtypes = [D, p, p, p, p, p, p]
        L.moe_load_stats.restype = i32
        L.moe_load_stats.argtypes = [D, p, p, p, p, p, sz, p]
        L.moe_quantize_fp8.restype = i32
        L.moe_quantize_fp8.argtypes = [C.c_int64, i32, i32, p, p, p, p]
        L.moe_expert_ffn_fp8.restype = i32
        L.moe_expert_ffn_fp8.argtypes = [D, p, p, p, p, p, p, p, p, p, p, sz, p]
        L.moe_layer_forward_fp8.restype = i32
        L.moe_layer_forward_fp8.argtypes = [D] + [p] * 16 + [C.POINTER(MoeDebugOut), p, sz, p]
        L.moe_quantize_mxfp4.restype = i32
        L.moe_quantize_mxfp4.argtypes = [C.c_int64, i32, i32, p, p, p, p]
        L.moe_expert_ffn_mxfp4.restype = i32
        L.moe_expert_ffn_mxfp4.argtypes = [D, p, p, p, p, p, p, p, p, p, p, sz, p]
        L.moe_layer_forward_mxfp4.restype = i32
        L.moe_layer_forward_mxfp4.argtypes = [D] + [p] * 16 + [C.POINTER(MoeDebugOut), p, sz, p]
        L.moe_quantize_mxfp8.restype = i32
        L.moe_quantize_mxfp8.argtypes = [C.c_int64, i32, i32, p, p, p, p]
        L.moe_expert_ffn_w4a8.restype = i32
        L.moe_expert_ffn_w4a8.argtypes = [D, p, p, p, p, p, p, p, p, p, p, sz, p]
        L.moe_layer_forward_w4a8.restype = i32
        L.moe_layer_forward_w4a8.argtypes = [D] + [p] * 16 + [C.POINTER(MoeDebugOut), p, sz, p]
        L.moe_cache_pool_bytes_mxfp4.restype = sz
        L.moe_cache_pool_bytes_mxfp4.argtypes = [D, i32]
        L.moe_cache_create_mxfp4.restype = i32
        L.moe_cache_create_mxfp4.argtypes = [D, i32, p, p, p, p, p, p, p, sz, C.POINTER(p)]
        L.moe_layer_forward_cached_w4a8.restype = i32
        L.moe_layer_forward_cached_w4a8.argtypes = [D, p, p, p, p] + [p] * 7 + [
            C.POINTER(MoeDebugOut), p, sz, p, p, C.POINTER(MoeCacheStep)]
        L.moe_cache_pool_bytes.restype = sz
        L.moe_cache_pool_bytes.argtypes = [D, i32]
        L.moe_cache_create.restype = i32
        L.moe_cache_create.argtypes = [D, i32, p, p, p, p, sz, C.POINTER(p)]
        L.moe_cache_destroy.restype = None
        L.moe_cache_destroy.argtypes = [p]
        L.moe_cache_load.restype = i32
        L.moe_cache_load.argtypes = [p, p, i32, p, p, C.POINTER(MoeCacheStep)]
        L.moe_cache_last_step.restype = i32
        L.moe_cache_last_step.argtypes = [p, C.POINTER(MoeCacheStep)]
        L.moe_cache_slots.restype = i32
        L.moe_cache_slots.argtypes = [p, p]
        L.moe_layer_forward_cached.restype = i32
        L.moe_layer_forward_cached.argtypes = [D, p, p, p, p, p, p, p, p, C.POINTER(MoeDebugOut),
                                               p, sz, p, p, C.POINTER(MoeCacheStep)]
        L.moe_layer_forward.restype = i32
        L.moe_layer_forward.argtypes = [D, p, p, p, p, p, p, p, p, p, p, C.POINTER(MoeDebugOut), p,
                                        sz, p]
        L.moe_static_scratch_bytes.restype = sz
        L.moe_static_scratch_bytes.argtypes = []
        L.moe_layer_forward_static.restype = i32
        L.moe_layer_forward_static.argtypes = [D, p, p, p, p, p, p, p, p, p, p,
                                               C.POINTER(MoeDebugOut), p]
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().moe_status_str(int(s)).decode()
