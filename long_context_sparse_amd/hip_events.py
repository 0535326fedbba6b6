"""HIP events without the system-scope release, for timing and for ordering
work across streams.

An event created with hipEventDisableSystemFence ends its marker with an
agent-scope release only.  Kernels on one GPU see each other's results
through that (a kernel's own completion already releases at agent scope);
the default system-scope release, which only host readers need, costs about
2.5 us per event pair on MI355X."""
from __future__ import annotations

import ctypes

_HIP = None
DISABLE_TIMING = 0x2
DISABLE_SYSTEM_FENCE = 0x20000000


def _rt():
    global _HIP
    if _HIP is None:
        import torch  # noqa: F401  (loads the HIP runtime that torch and the library share)
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        _HIP = h
    return _HIP


def _handle(stream):
    """Raw stream handle: a torch stream, an int handle, or None (torch's current stream)."""
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


class HipEvent:
    """A HIP event without the system fence; `timing=False` for pure ordering."""

    def __init__(self, timing: bool = True):
        self.h = ctypes.c_void_p()
        flags = DISABLE_SYSTEM_FENCE | (0 if timing else DISABLE_TIMING)
        rc = _rt().hipEventCreateWithFlags(ctypes.byref(self.h), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        rc = _rt().hipEventRecord(self.h, _handle(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream=None):
        """Make `stream` (default: torch's current stream) wait for this event."""
        rc = _rt().hipStreamWaitEvent(_handle(stream), self.h, 0)
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        f = ctypes.c_float()
        rc = _rt().hipEventElapsedTime(ctypes.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        if _HIP is not None and self.h:
            _HIP.hipEventDestroy(self.h)
