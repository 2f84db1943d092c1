"""Kernel timing through the library's w4a4_time_next_launch hook.

HIP events come from the HIP runtime that torch has already loaded (same
soname as the one libw4a4.so links), created and destroyed through ctypes.
An armed pair receives the start and end timestamps of the kernel the next
entry-point call launches, so elapsed() is that kernel's device duration.
"""
from __future__ import annotations

import ctypes

from . import _lib


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._live = []

    def create(self) -> ctypes.c_void_p:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self._live.append(e)
        return e

    def pair(self):
        return self.create(), self.create()

    @staticmethod
    def arm(start, stop) -> None:
        """Attach (start, stop) to the kernel of the next entry-point call on this thread."""
        if _lib.call("w4a4_time_next_launch", start, stop) != _lib.W4A4_OK:
            raise RuntimeError(_lib.last_error())

    def elapsed(self, start, stop) -> float:
        """Milliseconds between the two events (waits for the stop event)."""
        if self.hip.hipEventSynchronize(stop) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), start, stop) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self) -> None:
        for e in self._live:
            self.hip.hipEventDestroy(e)
        self._live = []
