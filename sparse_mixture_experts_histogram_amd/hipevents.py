"""hipEvent handles for timing the library's launches on their own stream.

Uses the HIP runtime already loaded in the process (the one torch and the
library share), so events and streams belong to the same runtime.
"""
from __future__ import annotations

import ctypes
import os
from typing import List

_hip = None


def hip():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the HIP runtime first)
        mode = getattr(os, "RTLD_NOLOAD", 4) | getattr(os, "RTLD_GLOBAL", 0)
        try:
            _hip = ctypes.CDLL("libamdhip64.so.7", mode=mode)
        except OSError:
            _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
    return _hip


class Events:
    """n raw hipEvents (created with default flags, so they record timing)."""

    def __init__(self, n: int):
        self.ev: List[ctypes.c_void_p] = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if hip().hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)
        self.array = (ctypes.c_void_p * n)(*[e.value for e in self.ev])

    def slice(self, start: int, n: int):
        """Pointer to events[start:start+n] as a void** for the C ABI."""
        return ctypes.cast(ctypes.byref(self.array, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.c_void_p)

    def ms(self, i: int, j: int) -> float:
        out = ctypes.c_float()
        hip().hipEventSynchronize(self.ev[j])
        if hip().hipEventElapsedTime(ctypes.byref(out), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.ev:
            hip().hipEventDestroy(e)
        self.ev = []
