"""Helpers of the GPU parity tests (no GPU work at import time)."""
import sys

import numpy as np


def say(msg: str):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if a.dtype == np.uint64:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).cuda().view(torch.uint64)
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.uint16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.uint64:
        return t.view(torch.int64).cpu().numpy().view(np.uint64)
    if t.dtype == torch.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    if a.shape != b.shape:
        return "shape %s vs %s" % (a.shape, b.shape)
    bad = np.argwhere(a != b)
    if len(bad) == 0:
        return "equal"
    i = tuple(bad[0])
    return "%d mismatches, first at %s: %r vs %r" % (len(bad), i, a[i], b[i])


class HipEvent:
    """A raw hipEvent_t from the HIP runtime torch has loaded (for the timed
    scan entry point): handle in .h, elapsed_ms(other) after a synchronize."""
    _lib = None

    @classmethod
    def _hip(cls):
        import ctypes
        if cls._lib is None:
            path = next(line.split()[-1] for line in open("/proc/self/maps")
                        if "libamdhip64" in line)
            lib = ctypes.CDLL(path)
            P = ctypes.c_void_p
            lib.hipEventCreate.argtypes = [ctypes.POINTER(P)]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
            lib.hipEventDestroy.argtypes = [P]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self.h = ctypes.c_void_p()
        assert self._hip().hipEventCreate(ctypes.byref(self.h)) == 0

    def elapsed_ms(self, other) -> float:
        import ctypes
        ms = ctypes.c_float()
        assert self._hip().hipEventElapsedTime(ctypes.byref(ms), self.h, other.h) == 0
        return ms.value

    def __del__(self):
        if self.h and HipEvent._lib is not None:
            HipEvent._lib.hipEventDestroy(self.h)
