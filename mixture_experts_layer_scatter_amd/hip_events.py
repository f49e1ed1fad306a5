"""Raw HIP events through the HIP runtime's C API (ctypes), for per-stage timing
of moe_layer_forward on the stream its kernels run on."""
from __future__ import annotations

import ctypes as C

_hip = None


def hip():
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        h.hipEventCreate.restype = C.c_int
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventDestroy.restype = C.c_int
        h.hipEventSynchronize.argtypes = [C.c_void_p]
        h.hipEventSynchronize.restype = C.c_int
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        h.hipEventElapsedTime.restype = C.c_int
        h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        h.hipEventRecord.restype = C.c_int
        _hip = h
    return _hip


class Event:
    def __init__(self):
        self.handle = C.c_void_p()
        if hip().hipEventCreate(C.byref(self.handle)) != 0:
            raise RuntimeError("hipEventCreate failed")

    def record(self, stream_handle):
        if hip().hipEventRecord(self.handle, C.c_void_p(stream_handle)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if hip().hipEventSynchronize(self.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_ms(self, end: "Event") -> float:
        ms = C.c_float()
        if hip().hipEventElapsedTime(C.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            if self.handle:
                hip().hipEventDestroy(self.handle)
        except Exception:
            pass
