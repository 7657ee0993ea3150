"""ctypes binding of libfathom.so: the calls of include/fathom.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are passed to
the C ABI, and a non-zero status raises FathomError.  Every step of the path
runs in the library's HIP kernels; there is no fallback of any kind.  Loading
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfathom.so")
_lock = threading.Lock()
_lib = None

BLOCK = 64
PLANES = 4
D = 128

STATUS = {
    0: "FATHOM_OK",
    -1: "FATHOM_ERR_NULL_ARG",
    -2: "FATHOM_ERR_BAD_SHAPE",
    -3: "FATHOM_ERR_BAD_RANGE",
    -4: "FATHOM_ERR_WORKSPACE",
    -5: "FATHOM_ERR_HIP",
    -6: "FATHOM_ERR_NO_DEVICE",
    -7: "FATHOM_ERR_ALIGNMENT",
    -8: "FATHOM_ERR_NOT_PINNED",
    -9: "FATHOM_ERR_TOO_LARGE",
}

EXPORTED = ("fathom_encode", "fathom_plan", "fathom_append_plan", "fathom_plan_fixed", "fathom_scan",
            "fathom_scan_timed", "fathom_topk",
            "fathom_scan_topk", "fathom_scan_topk_workspace_bytes", "fathom_gather",
            "fathom_klt_fit", "fathom_klt_fit_workspace_bytes", "fathom_klt_rotate_keys",
            "fathom_klt_rotate_queries",
            "fathom_topk_workspace_bytes", "fathom_topk_noalloc", "fathom_topk_noalloc_max_bytes",
            "fathom_test_cut_hooks", "fathom_status_string", "fathom_abi_version")


class FathomError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = lib().fathom_status_string(status).decode()
        super().__init__("%s failed: %s (%d)" % (where, name, status))


def lib():
    """The loaded libfathom.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libfathom.so is not built (run python -m "
                              "sparse_top_kv_fathom_amd.build); no fallback exists")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.fathom_encode.argtypes = [P, I64, I64, I32, I64, I64, P, P, P, P]
        L.fathom_plan.argtypes = [P, P, I64, I32, I32, I32, P, P, P, P]
        L.fathom_append_plan.argtypes = [P, I64, I64, I32, I64, I64, P, P, P, P, P, I32, I32, P,
                                         P, P, P]
        L.fathom_plan_fixed.argtypes = [P, P, I64, I32, I32, I32, I32, P, P]
        L.fathom_scan.argtypes = [P, P, I64, P, P, I64, I32, I32, I64, P, P]
        L.fathom_scan_timed.argtypes = [P, P, I64, P, P, I64, I32, I32, I64, P, P, P, P]
        L.fathom_topk.argtypes = [P, I64, I64, I32, P, P, SZ, P]
        L.fathom_topk_workspace_bytes.argtypes = [I64, I64, I32]
        L.fathom_topk_noalloc.argtypes = [P, I64, I64, I32, P, P]
        L.fathom_topk_noalloc_max_bytes.argtypes = []
        L.fathom_topk_noalloc_max_bytes.restype = SZ
        L.fathom_scan_topk.argtypes = [P, P, I64, P, P, I64, I32, I32, I64, I32, P, P, P, SZ, P]
        L.fathom_scan_topk_workspace_bytes.argtypes = [I64, I32, I64, I32]
        L.fathom_scan_topk_workspace_bytes.restype = SZ
        L.fathom_gather.argtypes = [P, P, I64, P, I64, I32, I64, P, P, P]
        L.fathom_klt_fit_workspace_bytes.argtypes = [I64, I64, I32]
        L.fathom_klt_fit_workspace_bytes.restype = SZ
        L.fathom_klt_fit.argtypes = [P, I64, I64, I32, P, P, P, P, SZ, P]
        L.fathom_klt_rotate_keys.argtypes = [P, P, P, I64, I64, I32, P, P]
        L.fathom_klt_rotate_queries.argtypes = [P, P, I64, I32, I32, P, P]
        L.fathom_topk_workspace_bytes.restype = SZ
        L.fathom_status_string.argtypes = [ctypes.c_int]
        L.fathom_status_string.restype = ctypes.c_char_p
        L.fathom_abi_version.argtypes = []
        for f in ("fathom_encode", "fathom_plan", "fathom_plan_fixed", "fathom_scan",
                  "fathom_scan_timed", "fathom_topk",
                  "fathom_scan_topk", "fathom_gather", "fathom_klt_fit",
                  "fathom_klt_rotate_keys", "fathom_klt_rotate_queries", "fathom_abi_version"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
        return L


def _check(status: int, where: str):
    if status != 0:
        raise FathomError(status, where)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


def _opt(t, name, dtype, shape):
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtype, shape)


def store_shapes(groups: int, nb_store: int, d: int = D):
    """Shapes of the plane and scale arrays of a store of nb_store blocks."""
    return (groups, d, PLANES, nb_store), (groups, d, nb_store)


def empty_store(groups: int, nb_store: int, device="cuda", d: int = D):
    ps, ss = store_shapes(groups, nb_store, d)
    return (torch.empty(ps, dtype=torch.uint64, device=device),
            torch.empty(ss, dtype=torch.uint16, device=device))


def encode(k: torch.Tensor, planes: torch.Tensor | None = None, scales: torch.Tensor | None = None,
           block_offset: int = 0, nonfinite_flag: torch.Tensor | None = None, stream=None):
    """fathom_encode: k [groups][n][d] fp16 -> (planes, scales).  Writes block
    slots [block_offset, block_offset + n/64) of the given store (a new store
    of exactly n/64 blocks when planes/scales are None)."""
    groups, n, d = k.shape
    if planes is None:
        planes, scales = empty_store(groups, n // BLOCK, k.device, d)
    nb_store = planes.shape[-1]
    ps, ss = store_shapes(groups, nb_store, d)
    st = lib().fathom_encode(
        _dev(k, "k", torch.float16), groups, n, d, nb_store, block_offset,
        _dev(planes, "planes", torch.uint64, ps), _dev(scales, "scales", torch.uint16, ss),
        _opt(nonfinite_flag, "nonfinite_flag", torch.int32, (1,)), _stream(stream))
    _check(st, "fathom_encode")
    return planes, scales


def plan(q: torch.Tensor, var: torch.Tensor, budget_bits: int, depths: torch.Tensor | None = None,
         theta: torch.Tensor | None = None, bits_used: torch.Tensor | None = None, stream=None):
    """fathom_plan: q [groups][G][d] fp32, var [groups][d] fp32 -> depths uint8 [groups][d]."""
    groups, G, d = q.shape
    if depths is None:
        depths = torch.empty((groups, d), dtype=torch.uint8, device=q.device)
    st = lib().fathom_plan(
        _dev(q, "q", torch.float32), _dev(var, "var", torch.float32, (groups, d)), groups, G, d,
        int(budget_bits), _dev(depths, "depths", torch.uint8, (groups, d)),
        _opt(theta, "theta", torch.float64, (groups,)),
        _opt(bits_used, "bits_used", torch.int32, (groups,)), _stream(stream))
    _check(st, "fathom_plan")
    return depths


def append_plan(k: torch.Tensor, planes: torch.Tensor, scales: torch.Tensor, block_offset: int,
                q: torch.Tensor, var: torch.Tensor, budget_bits: int,
                depths: torch.Tensor | None = None, theta: torch.Tensor | None = None,
                bits_used: torch.Tensor | None = None, nonfinite_flag: torch.Tensor | None = None,
                stream=None):
    """fathom_append_plan: encode(k, planes, scales, block_offset) and
    plan(q, var, budget_bits) in one call (one launch for an append of at
    most 64 blocks per group) -> depths uint8 [groups][d]."""
    groups, n, d = k.shape
    G = q.shape[1]
    nb_store = planes.shape[-1]
    ps, ss = store_shapes(groups, nb_store, d)
    if depths is None:
        depths = torch.empty((groups, d), dtype=torch.uint8, device=q.device)
    st = lib().fathom_append_plan(
        _dev(k, "k", torch.float16), groups, n, d, nb_store, block_offset,
        _dev(planes, "planes", torch.uint64, ps), _dev(scales, "scales", torch.uint16, ss),
        _opt(nonfinite_flag, "nonfinite_flag", torch.int32, (1,)),
        _dev(q, "q", torch.float32, (groups, G, d)), _dev(var, "var", torch.float32, (groups, d)),
        G, int(budget_bits), _dev(depths, "depths", torch.uint8, (groups, d)),
        _opt(theta, "theta", torch.float64, (groups,)),
        _opt(bits_used, "bits_used", torch.int32, (groups,)), _stream(stream))
    _check(st, "fathom_append_plan")
    return depths


PLAN_MODES = {"uniform": 1, "sparq": 2, "topstat": 3}


def plan_fixed(mode: str, param: int, q: torch.Tensor | None = None,
               stat: torch.Tensor | None = None, groups: int | None = None, G: int | None = None,
               depths: torch.Tensor | None = None, stream=None):
    """fathom_plan_fixed: 'uniform' (every channel at depth param), 'sparq'
    (depth 4 on the param channels with the largest sum_h |q_hj|) or 'topstat'
    (the same ranked by stat [groups][d]) -> depths uint8 [groups][d]."""
    if q is not None:
        groups, G, d = q.shape
        device = q.device
    elif stat is not None:
        groups, d = stat.shape
        G = G or 1
        device = stat.device
    else:
        d = 128
        device = depths.device if depths is not None else torch.device("cuda")
    if depths is None:
        depths = torch.empty((groups, d), dtype=torch.uint8, device=device)
    st = lib().fathom_plan_fixed(
        _opt(q, "q", torch.float32, (groups, G, d)), _opt(stat, "stat", torch.float32, (groups, d)),
        groups, G, d, PLAN_MODES[mode], int(param),
        _dev(depths, "depths", torch.uint8, (groups, d)), _stream(stream))
    _check(st, "fathom_plan_fixed")
    return depths


def scan(planes: torch.Tensor, scales: torch.Tensor, depths: torch.Tensor, q: torch.Tensor,
         n: int, scores: torch.Tensor | None = None, stream=None, events=None):
    """fathom_scan: scores [groups][G][n] fp32 of the first n keys of the store.

    events: None, or (start, stop) raw hipEvent_t handles (ints or
    ctypes.c_void_p) that fathom_scan_timed records from the scan kernels' own
    start and end timestamps."""
    groups, G, d = q.shape
    nb_store = planes.shape[-1]
    ps, ss = store_shapes(groups, nb_store, d)
    if scores is None:
        scores = torch.empty((groups, G, n), dtype=torch.float32, device=q.device)
    args = (_dev(planes, "planes", torch.uint64, ps), _dev(scales, "scales", torch.uint16, ss),
            nb_store, _dev(depths, "depths", torch.uint8, (groups, d)),
            _dev(q, "q", torch.float32), groups, G, d, int(n),
            _dev(scores, "scores", torch.float32, (groups, G, n)))
    if events is None:
        st = lib().fathom_scan(*args, _stream(stream))
        _check(st, "fathom_scan")
    else:
        e0, e1 = (e if isinstance(e, ctypes.c_void_p) else ctypes.c_void_p(e) for e in events)
        st = lib().fathom_scan_timed(*args, e0, e1, _stream(stream))
        _check(st, "fathom_scan_timed")
    return scores


def gather(host_planes: torch.Tensor, host_scales: torch.Tensor, depths: torch.Tensor, n: int,
           planes: torch.Tensor, scales: torch.Tensor, stream=None):
    """fathom_gather: the runs `depths` reads, blocks [0, n/64), from a pinned
    host store into the device store (same layout)."""
    groups, d, _, nb_store = planes.shape
    ps, ss = store_shapes(groups, nb_store, d)
    for t, name in ((host_planes, "host_planes"), (host_scales, "host_scales")):
        if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
            raise ValueError("%s must be a contiguous pinned host tensor" % name)
    if tuple(host_planes.shape) != ps or tuple(host_scales.shape) != ss:
        raise ValueError("host store shapes must match the device store")
    st = lib().fathom_gather(
        ctypes.c_void_p(host_planes.data_ptr()), ctypes.c_void_p(host_scales.data_ptr()), nb_store,
        _dev(depths, "depths", torch.uint8, (groups, d)), groups, d, int(n),
        _dev(planes, "planes", torch.uint64, ps), _dev(scales, "scales", torch.uint16, ss),
        _stream(stream))
    _check(st, "fathom_gather")
    return planes, scales


def test_cut_hooks(publish: bool = True, spin_limit: int = 2048) -> None:
    """fathom_test_cut_hooks (tests of fathom_scan_topk's fallback only)."""
    _check(lib().fathom_test_cut_hooks(int(bool(publish)), int(spin_limit)),
           "fathom_test_cut_hooks")


def scan_topk_workspace(groups: int, G: int, n: int, k: int, device="cuda") -> torch.Tensor:
    nbytes = int(lib().fathom_scan_topk_workspace_bytes(groups, G, n, k))
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def scan_topk(planes: torch.Tensor, scales: torch.Tensor, depths: torch.Tensor, q: torch.Tensor,
              n: int, k: int, scores: torch.Tensor | None = None,
              indices: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
              stream=None, write_scores: bool = True):
    """fathom_scan_topk: (scores [groups][G][n] fp32 or None, indices
    [groups*G][k] int32).  write_scores=False passes no score buffer (the
    scores are then not returned)."""
    groups, G, d = q.shape
    nb_store = planes.shape[-1]
    ps, ss = store_shapes(groups, nb_store, d)
    if not write_scores:
        scores = None
    elif scores is None:
        scores = torch.empty((groups, G, n), dtype=torch.float32, device=q.device)
    if indices is None:
        indices = torch.empty((groups * G, k), dtype=torch.int32, device=q.device)
    if workspace is None:
        workspace = scan_topk_workspace(groups, G, n, k, q.device)
    st = lib().fathom_scan_topk(
        _dev(planes, "planes", torch.uint64, ps), _dev(scales, "scales", torch.uint16, ss),
        nb_store, _dev(depths, "depths", torch.uint8, (groups, d)), _dev(q, "q", torch.float32),
        groups, G, d, int(n), int(k), _opt(scores, "scores", torch.float32, (groups, G, n)),
        _dev(indices, "indices", torch.int32, (groups * G, k)),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(st, "fathom_scan_topk")
    return scores, indices


def topk_workspace_bytes(rows: int, n: int, k: int) -> int:
    return int(lib().fathom_topk_workspace_bytes(rows, n, k))


def topk_workspace(rows: int, n: int, k: int, device="cuda") -> torch.Tensor:
    nbytes = topk_workspace_bytes(rows, n, k)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def topk(scores: torch.Tensor, k: int, indices: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream=None):
    """fathom_topk: scores [..., n] fp32 -> indices [rows][k] int32 ascending."""
    n = scores.shape[-1]
    rows = scores.numel() // n
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    if workspace is None:
        workspace = topk_workspace(rows, n, k, scores.device)
    st = lib().fathom_topk(
        _dev(scores, "scores", torch.float32), rows, n, int(k),
        _dev(indices, "indices", torch.int32, (rows, k)), _dev(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream))
    _check(st, "fathom_topk")
    return indices


def topk_noalloc(scores: torch.Tensor, k: int, indices: torch.Tensor, stream=None):
    """fathom_topk_noalloc: fathom_topk with the library's fixed scratch as
    its workspace (the call allocates nothing; `indices` [rows][k] int32 is
    the caller's)."""
    n = scores.shape[-1]
    rows = scores.numel() // n
    st = lib().fathom_topk_noalloc(
        _dev(scores, "scores", torch.float32), rows, n, int(k),
        _dev(indices, "indices", torch.int32, (rows, k)), _stream(stream))
    _check(st, "fathom_topk_noalloc")
    return indices


def klt_fit_workspace(groups: int, n: int, device="cuda") -> torch.Tensor:
    nbytes = int(lib().fathom_klt_fit_workspace_bytes(groups, n, D))
    if nbytes == 0:
        raise ValueError("invalid shape for fathom_klt_fit (groups=%d, n=%d)" % (groups, n))
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def klt_fit(k: torch.Tensor, workspace: torch.Tensor | None = None, stream=None):
    """fathom_klt_fit: k [groups][n][d] fp16 -> (mu [groups][d], basis
    [groups][d][d], lam [groups][d]), fp32."""
    groups, n, d = k.shape
    mu = torch.empty((groups, d), dtype=torch.float32, device=k.device)
    basis = torch.empty((groups, d, d), dtype=torch.float32, device=k.device)
    lam = torch.empty((groups, d), dtype=torch.float32, device=k.device)
    if workspace is None:
        workspace = klt_fit_workspace(groups, n, k.device)
    st = lib().fathom_klt_fit(_dev(k, "k", torch.float16), groups, n, d, _dev(mu, "mu", torch.float32),
                              _dev(basis, "basis", torch.float32), _dev(lam, "lam", torch.float32),
                              _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                              _stream(stream))
    _check(st, "fathom_klt_fit")
    return mu, basis, lam


def klt_rotate_keys(k: torch.Tensor, mu: torch.Tensor, basis: torch.Tensor,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fathom_klt_rotate_keys: (k - mu) basis, binary16 [groups][n][d]."""
    groups, n, d = k.shape
    if out is None:
        out = torch.empty_like(k)
    st = lib().fathom_klt_rotate_keys(
        _dev(k, "k", torch.float16), _dev(mu, "mu", torch.float32, (groups, d)),
        _dev(basis, "basis", torch.float32, (groups, d, d)), groups, n, d,
        _dev(out, "out", torch.float16, (groups, n, d)), _stream(stream))
    _check(st, "fathom_klt_rotate_keys")
    return out


def klt_rotate_queries(q: torch.Tensor, basis: torch.Tensor, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """fathom_klt_rotate_queries: q basis, fp32 [groups][G][d]."""
    groups, G, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    st = lib().fathom_klt_rotate_queries(
        _dev(q, "q", torch.float32), _dev(basis, "basis", torch.float32, (groups, d, d)), groups,
        G, d, _dev(out, "out", torch.float32, (groups, G, d)), _stream(stream))
    _check(st, "fathom_klt_rotate_queries")
    return out
