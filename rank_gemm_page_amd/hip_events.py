"""Raw HIP events through ctypes (timing plumbing for slora_lora_delta_timed)."""
from __future__ import annotations

import ctypes
import os

_HIP = None


def _hip():
    """The HIP runtime already in the process (the one torch and libslora use)."""
    global _HIP
    if _HIP is None:
        try:
            _HIP = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_LAZY)
        except OSError:
            _HIP = ctypes.CDLL("libamdhip64.so.7")
        _HIP.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _HIP.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _HIP


class HipEvent:
    """A timing-enabled hipEvent_t owned by Python."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = _hip().hipEventCreate(ctypes.byref(h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.handle = h.value

    def synchronize(self):
        rc = _hip().hipEventSynchronize(self.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = _hip().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and _HIP is not None:
            _HIP.hipEventDestroy(self.handle)
            self.handle = None
