"""HIP events through ctypes on libamdhip64, for the library's timing hook.

torch creates its event handles lazily (at the first torch-side record), so
raw hipEvent_t handles are made here instead and passed to the library,
which records them on the launch stream.
"""
from __future__ import annotations

import ctypes
import ctypes.util

_hip = None


def _lib():
    global _hip
    if _hip is None:
        name = ctypes.util.find_library("amdhip64") or "libamdhip64.so"
        for cand in (name, "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(cand)
                break
            except OSError:
                continue
        if _hip is None:
            raise RuntimeError("libamdhip64.so not found")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    return _hip


class HipEvent:
    """One hipEvent_t; `.cuda_event` is the raw handle the library records."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = _lib().hipEventCreate(ctypes.byref(h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.cuda_event = h.value

    def synchronize(self):
        rc = _lib().hipEventSynchronize(ctypes.c_void_p(self.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_time(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _lib().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                        ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "cuda_event", None) and _hip is not None:
            _hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))
            self.cuda_event = None
