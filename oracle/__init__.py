"""CPU oracle of the Fathom key scan — test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package never imports the product.

The arithmetic lives in ``fathom_oracle.c`` (plain C, fp64 except for the
fp32 evaluation orders reproduced on purpose: the scan's, and the rotation
folds of the KLT-rotated store) and, for the KLT fit, in numpy fp64 with its
symmetric eigensolver.  This module compiles it with
gcc on first use and wraps it for numpy arrays.  Each wrapper names the
passage of "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
Caches" (papers.paperslantern.ai/papers/2609.17652 and the jaehun.me review)
that the C function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fathom_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfathom_oracle.so")
_lock = threading.Lock()
_lib = None

BLOCK = 64
PLANES = 4


def build(force: bool = False) -> str:
    """Compile fathom_oracle.c into libfathom_oracle.so (gcc, -O2, no FP contraction)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # FATHOM_ORACLE_LIB: a build of fathom_oracle.c made elsewhere (the
        # sanitizer test's instrumented one) instead of the default build.
        lib = ctypes.CDLL(os.environ.get("FATHOM_ORACLE_LIB") or build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.fo_encode.argtypes = [P, I64, I64, I, I64, I64, P, P, I]
        lib.fo_encode.restype = I64
        lib.fo_decode.argtypes = [P, P, I64, I64, I, I64, I, P]
        lib.fo_decode.restype = None
        lib.fo_dequant.argtypes = [ctypes.c_uint16, I, I]
        lib.fo_dequant.restype = ctypes.c_double
        lib.fo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.fo_f16_to_f64.restype = ctypes.c_double
        lib.fo_importance.argtypes = [P, P, I, I, P]
        lib.fo_importance.restype = None
        lib.fo_depth_one.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.fo_depth_one.restype = I
        lib.fo_depths_at.argtypes = [P, I, ctypes.c_double, P]
        lib.fo_depths_at.restype = I
        lib.fo_bisect.argtypes = [P, I, I, ctypes.c_double, ctypes.c_double, I, P, P, P]
        lib.fo_bisect.restype = None
        lib.fo_plan_group.argtypes = [P, I, I, P, P, P]
        lib.fo_plan_group.restype = None
        lib.fo_plan.argtypes = [P, P, I64, I, I, I, P, P, P, I]
        lib.fo_plan.restype = None
        lib.fo_scan_f64.argtypes = [P, P, I64, P, P, I64, I, I, I64, P, P, I]
        lib.fo_scan_f64.restype = None
        lib.fo_scan_ref32.argtypes = [P, P, I64, P, P, I64, I, I, I64, P, I]
        lib.fo_scan_ref32.restype = None
        lib.fo_topk.argtypes = [P, I64, I64, I, P, I]
        lib.fo_topk.restype = None
        lib.fo_klt_rotate.argtypes = [P, P, P, I64, I64, I, P, I]
        lib.fo_klt_rotate.restype = None
        lib.fo_klt_rotate_q.argtypes = [P, P, I64, I, I, P]
        lib.fo_klt_rotate_q.restype = None
        lib.fo_max_threads.argtypes = []
        lib.fo_max_threads.restype = I
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def max_threads() -> int:
    return int(_load().fo_max_threads())


# --------------------------------------------------------------------------
# Encode — §3.2 "Bit-Plane K Cache"
# --------------------------------------------------------------------------

def encode(k_f16: np.ndarray, nb_store: int | None = None, block_offset: int = 0,
           planes: np.ndarray | None = None, scales: np.ndarray | None = None,
           nthreads: int = 0):
    """fp16 keys [groups][n][d] -> (planes [groups][d][4][nb_store] uint64,
    scales [groups][d][nb_store] uint16 (fp16 bits of the block max a),
    number of blocks holding a non-finite value).  §3.2."""
    k = np.ascontiguousarray(k_f16)
    if k.dtype == np.float16:
        k = k.view(np.uint16)
    assert k.dtype == np.uint16 and k.ndim == 3
    groups, n, d = k.shape
    assert n % BLOCK == 0
    nb = n // BLOCK
    if nb_store is None:
        nb_store = nb
    assert block_offset + nb <= nb_store
    if planes is None:
        planes = np.zeros((groups, d, PLANES, nb_store), dtype=np.uint64)
    if scales is None:
        scales = np.zeros((groups, d, nb_store), dtype=np.uint16)
    bad = _load().fo_encode(_ptr(k), groups, n, d, nb_store, block_offset,
                            _ptr(planes), _ptr(scales), int(nthreads or max_threads()))
    return planes, scales, int(bad)


def decode(planes: np.ndarray, scales: np.ndarray, n: int, t: int) -> np.ndarray:
    """Every token read back at uniform depth t (fp64, [groups][n][d]):
    (c >> (4-t) + 0.5 - 2^(t-1)) * a / 2^(t-1).  §3.2."""
    groups, d, _, nb_store = planes.shape
    out = np.zeros((groups, n, d), dtype=np.float64)
    _load().fo_decode(_ptr(planes), _ptr(scales), groups, n, d, nb_store, t, _ptr(out))
    return out


def dequant(a_bits: int, cprefix: int, t: int) -> float:
    """One prefix value (§3.2)."""
    return float(_load().fo_dequant(a_bits, cprefix, t))


def f16_to_f64(bits: int) -> float:
    return float(_load().fo_f16_to_f64(bits))


# --------------------------------------------------------------------------
# Plan — §3.3 "Per-Query Read Depth", Eq. 4; Appendix A
# --------------------------------------------------------------------------

def importance(q: np.ndarray, var: np.ndarray) -> np.ndarray:
    """g_j = sum_h q_hj^2 * Var_j in fp64 for one group; q [G][d], var [d]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    var = np.ascontiguousarray(var, dtype=np.float32)
    G, d = q.shape
    g = np.zeros(d, dtype=np.float64)
    _load().fo_importance(_ptr(q), _ptr(var), G, d, _ptr(g))
    return g


def depth_one(g: float, theta: float) -> int:
    return int(_load().fo_depth_one(float(g), float(theta)))


def depths_at(g: np.ndarray, theta: float):
    """(depths, sum) at water line theta (Eq. 4 with halves rounded up)."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    t = np.zeros(g.shape[0], dtype=np.uint8)
    s = _load().fo_depths_at(_ptr(g), g.shape[0], float(theta), _ptr(t))
    return t, int(s)


def bisect(g: np.ndarray, budget: int, lo: float, hi: float, steps: int = 30):
    """Log-bisection on a caller-given bracket (Appendix A uses [0.001, 10])."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    t = np.zeros(g.shape[0], dtype=np.uint8)
    th = ctypes.c_double()
    bits = ctypes.c_int()
    _load().fo_bisect(_ptr(g), g.shape[0], int(budget), float(lo), float(hi), int(steps),
                      _ptr(t), ctypes.byref(th), ctypes.byref(bits))
    return t, th.value, bits.value


def plan_group(g: np.ndarray, budget: int):
    """Plan of one group from its importances (general bracket)."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    t = np.zeros(g.shape[0], dtype=np.uint8)
    th = ctypes.c_double()
    bits = ctypes.c_int()
    _load().fo_plan_group(_ptr(g), g.shape[0], int(budget), _ptr(t), ctypes.byref(th),
                          ctypes.byref(bits))
    return t, th.value, bits.value


def plan(q: np.ndarray, var: np.ndarray, budget: int, nthreads: int = 0):
    """q [groups][G][d] fp32, var [groups][d] fp32 -> (depths uint8 [groups][d],
    theta fp64 [groups], bits int32 [groups])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    var = np.ascontiguousarray(var, dtype=np.float32)
    groups, G, d = q.shape
    depths = np.zeros((groups, d), dtype=np.uint8)
    theta = np.zeros(groups, dtype=np.float64)
    bits = np.zeros(groups, dtype=np.int32)
    _load().fo_plan(_ptr(q), _ptr(var), groups, G, d, int(budget), _ptr(depths),
                    _ptr(theta), _ptr(bits), int(nthreads or max_threads()))
    return depths, theta, bits


# --------------------------------------------------------------------------
# Fixed-depth plans — the §2 comparison points (2-bit thumbnail, SparQ,
# Double Sparsity's offline channel set) read through the same store
# --------------------------------------------------------------------------

def plan_fixed(mode: str, param: int, q=None, stat=None, groups=None, d: int = 128):
    """'uniform': every channel at depth `param` (the 2-bit thumbnail reads all
    channels at two planes).  'sparq': depth 4 on the `param` channels with the
    largest sum over the query heads of |q_hj| (SparQ's rule under grouped
    queries, the sum taken in fp64 head by head), 0 elsewhere.  'topstat': the
    same ranked by a given per-channel statistic (a fixed set chosen offline).
    Equal statistics rank by the lower channel index.  -> depths uint8
    [groups][d]."""
    if mode == "uniform":
        return np.full((groups, d), param, dtype=np.uint8)
    if mode == "sparq":
        q = np.asarray(q, dtype=np.float32)
        groups, G, d = q.shape
        s = np.zeros((groups, d), dtype=np.float64)
        for h in range(G):                      # heads in order, one rounding each
            s = s + np.abs(q[:, h, :].astype(np.float64))
    elif mode == "topstat":
        s = np.asarray(stat, dtype=np.float32).astype(np.float64)
        groups, d = s.shape
    else:
        raise ValueError(mode)
    depths = np.zeros((groups, d), dtype=np.uint8)
    j = np.arange(d)
    for g in range(groups):
        order = np.lexsort((j, -s[g]))          # statistic descending, then index
        depths[g, order[:param]] = 4
    return depths


# --------------------------------------------------------------------------
# Scan — §3.2 prefix dequantization over the §3.3 active channels
# --------------------------------------------------------------------------

def scan_f64(planes, scales, depths, q, n: int, nthreads: int = 0):
    """Plain fp64 scores S_hi = sum_{t_j>0} q_hj khat_ij and their L1 magnitude.
    Returns (scores [groups][G][n] fp64, l1 [groups][G][n] fp64)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    groups, G, d = q.shape
    nb_store = planes.shape[3]
    s = np.zeros((groups, G, n), dtype=np.float64)
    l1 = np.zeros((groups, G, n), dtype=np.float64)
    _load().fo_scan_f64(_ptr(planes), _ptr(scales), nb_store, _ptr(np.ascontiguousarray(depths)),
                        _ptr(q), groups, G, d, n, _ptr(s), _ptr(l1),
                        int(nthreads or max_threads()))
    return s, l1


def scan_ref32(planes, scales, depths, q, n: int, nthreads: int = 0):
    """Scores in the stated fp32 evaluation order ([groups][G][n] fp32)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    groups, G, d = q.shape
    nb_store = planes.shape[3]
    s = np.zeros((groups, G, n), dtype=np.float32)
    _load().fo_scan_ref32(_ptr(planes), _ptr(scales), nb_store,
                          _ptr(np.ascontiguousarray(depths)), _ptr(q), groups, G, d, n,
                          _ptr(s), int(nthreads or max_threads()))
    return s


# --------------------------------------------------------------------------
# Top-k — per query head (§2)
# --------------------------------------------------------------------------

def topk(scores: np.ndarray, k: int, nthreads: int = 0) -> np.ndarray:
    """scores [rows][n] fp32 -> indices [rows][k] int32, ascending; order of
    selection: score descending, lower index first on ties (full sort)."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    s2 = s.reshape(-1, s.shape[-1])
    rows, n = s2.shape
    assert 1 <= k <= n
    idx = np.zeros((rows, k), dtype=np.int32)
    _load().fo_topk(_ptr(s2), rows, n, int(k), _ptr(idx), int(nthreads or max_threads()))
    return idx


# ---------------------------------------------------------------------------
# KLT-rotated store (§3.5 "rotated variant"; Appendix D's calibration-free fit)
# ---------------------------------------------------------------------------

def klt_order_and_sign(lam: np.ndarray, V: np.ndarray):
    """Canonical eigenbasis: columns by eigenvalue descending (equal values
    keep their incoming order); in each column the first component of
    magnitude at least 1/(2 sqrt(d)) made positive (a unit vector always has
    one; a threshold well below the largest magnitude keeps the choice stable
    when several components are nearly equal); eigenvalues below 0, which a
    covariance cannot have, read as 0."""
    order = np.argsort(-lam, kind="stable")
    lam = np.maximum(lam[order], 0.0)
    V = V[:, order].copy()
    thr = 0.5 / np.sqrt(V.shape[0])
    for j in range(V.shape[1]):
        r = int(np.argmax(np.abs(V[:, j]) >= thr))
        if V[r, j] < 0:
            V[:, j] = -V[:, j]
    return lam, V


def klt_fit(k_f16: np.ndarray):
    """Per group: mean mu, covariance C = (k - mu)^T (k - mu) / (n - 1) of the
    binary16 keys, in fp64, and its eigenpairs (numpy's symmetric
    eigensolver), canonically ordered and signed.  The pages build the
    rotated store from the eigenbasis of the keys' covariance with its
    eigenvalues as the channel variances (§3.5), fitted once on calibration
    keys or, in the calibration-free variant, on the session's own keys
    (Appendix D).  Returns (mu [groups][d], V [groups][d][d] with eigenvector
    j in column j, lam [groups][d]), all fp64."""
    k = np.asarray(k_f16, dtype=np.float16)
    groups, n, d = k.shape
    mu = np.empty((groups, d))
    V = np.empty((groups, d, d))
    lam = np.empty((groups, d))
    for g in range(groups):
        x = k[g].astype(np.float64)
        mu[g] = x.sum(axis=0) / n
        xc = x - mu[g]
        C = (xc.T @ xc) / (n - 1)
        w, E = np.linalg.eigh(C)
        lam[g], V[g] = klt_order_and_sign(w, E)
    return mu, V, lam


def klt_rotate_keys(k_f16: np.ndarray, mu32: np.ndarray, V32: np.ndarray, nthreads: int = 0,
                    raw: bool = False):
    """Rotated keys (k - mu) V (§3.5), the fp32 fold of fo_klt_rotate rounded
    to binary16 nearest-even: the input of encode in the rotated variant.
    raw=True returns the fp32 fold before rounding."""
    k = np.ascontiguousarray(np.asarray(k_f16, dtype=np.float16))
    groups, n, d = k.shape
    mu = np.ascontiguousarray(mu32, dtype=np.float32)
    V = np.ascontiguousarray(V32, dtype=np.float32)
    assert mu.shape == (groups, d) and V.shape == (groups, d, d)
    out = np.empty((groups, n, d), dtype=np.float32)
    _load().fo_klt_rotate(_ptr(k.view(np.uint16)), _ptr(mu), _ptr(V), groups, n, d, _ptr(out),
                          nthreads or max_threads())
    return out if raw else out.astype(np.float16)


def klt_rotate_queries(q: np.ndarray, V32: np.ndarray):
    """Rotated queries q V (§3.5: the importance becomes sum_h ((q_h V)_j)^2
    lambda_j, i.e. the plan of the rotated queries with lambda as the
    variances), the fp32 fold of fo_klt_rotate_q."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    groups, G, d = q.shape
    V = np.ascontiguousarray(V32, dtype=np.float32)
    assert V.shape == (groups, d, d)
    out = np.empty_like(q)
    _load().fo_klt_rotate_q(_ptr(q), _ptr(V), groups, G, d, _ptr(out))
    return out
