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
