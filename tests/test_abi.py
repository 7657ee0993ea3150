"""The C-ABI library loads, exports every call include/fathom.h declares, and
rejects invalid arguments on the host before any HIP call (CPU only: fake
non-NULL pointers are never dereferenced because validation fails first)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fathom.h")
LIB = os.path.join(ROOT, "sparse_top_kv_fathom_amd", "libfathom.so")

OK, NULL_ARG, BAD_SHAPE, BAD_RANGE, WORKSPACE, HIP, NO_DEVICE, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7
P = ctypes.c_void_p
FAKE = P(1 << 20)           # a well-aligned, never dereferenced address


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fathom_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        import sparse_top_kv_fathom_amd.build as b
        b.build()
    import sparse_top_kv_fathom_amd as fk
    return fk.lib()


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_header_declares_the_calls():
    names = declared()
    for f in ("fathom_encode", "fathom_plan", "fathom_append_plan", "fathom_plan_fixed", "fathom_scan",
              "fathom_scan_timed", "fathom_topk",
              "fathom_scan_topk", "fathom_scan_topk_workspace_bytes", "fathom_gather",
              "fathom_klt_fit", "fathom_klt_fit_workspace_bytes", "fathom_klt_rotate_keys",
              "fathom_klt_rotate_queries",
              "fathom_topk_workspace_bytes", "fathom_topk_noalloc", "fathom_topk_noalloc_max_bytes",
              "fathom_test_cut_hooks", "fathom_status_string", "fathom_abi_version"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared():
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert L.fathom_abi_version() == 9
    for code in (OK, NULL_ARG, BAD_SHAPE, BAD_RANGE, WORKSPACE, HIP, NO_DEVICE, ALIGN, -8, -9):
        s = L.fathom_status_string(code).decode()
        assert s.startswith("FATHOM_")
    assert L.fathom_status_string(12345).decode() == "FATHOM_ERR_UNKNOWN"


def test_encode_validation(L):
    e = L.fathom_encode
    assert e(None, 1, 4096, 128, 64, 0, FAKE, FAKE, None, None) == NULL_ARG
    assert e(FAKE, 1, 4096, 128, 64, 0, None, FAKE, None, None) == NULL_ARG
    assert e(FAKE, 1, 4096, 64, 64, 0, FAKE, FAKE, None, None) == BAD_SHAPE      # d != 128
    assert e(FAKE, 0, 4096, 128, 64, 0, FAKE, FAKE, None, None) == BAD_SHAPE     # groups
    assert e(FAKE, 70000, 4096, 128, 64, 0, FAKE, FAKE, None, None) == BAD_SHAPE
    assert e(FAKE, 1, 4000, 128, 64, 0, FAKE, FAKE, None, None) == BAD_SHAPE     # n % 64
    assert e(FAKE, 1, 0, 128, 64, 0, FAKE, FAKE, None, None) == BAD_SHAPE        # empty
    assert e(FAKE, 1, 1 << 31, 128, 1 << 25, 0, FAKE, FAKE, None, None) == BAD_SHAPE
    assert e(FAKE, 1, 4096, 128, 63, 0, FAKE, FAKE, None, None) == BAD_SHAPE     # capacity
    assert e(FAKE, 1, 4096, 128, 70, 7, FAKE, FAKE, None, None) == BAD_SHAPE     # offset+nb
    assert e(FAKE, 1, 4096, 128, 70, -1, FAKE, FAKE, None, None) == BAD_SHAPE
    assert e(P(8), 1, 4096, 128, 64, 0, FAKE, FAKE, None, None) == ALIGN         # k 16 B
    assert e(FAKE, 1, 4096, 128, 64, 0, P(4), FAKE, None, None) == ALIGN
    assert e(FAKE, 1, 4096, 128, 64, 0, FAKE, FAKE, P(2), None) == ALIGN


def test_plan_validation(L):
    p = L.fathom_plan
    assert p(None, FAKE, 1, 4, 128, 92, FAKE, None, None, None) == NULL_ARG
    assert p(FAKE, FAKE, 1, 4, 128, 92, None, None, None, None) == NULL_ARG
    assert p(FAKE, FAKE, 1, 0, 128, 92, FAKE, None, None, None) == BAD_SHAPE
    assert p(FAKE, FAKE, 1, 9, 128, 92, FAKE, None, None, None) == BAD_SHAPE
    assert p(FAKE, FAKE, 1, 4, 100, 92, FAKE, None, None, None) == BAD_SHAPE
    assert p(FAKE, FAKE, 0, 4, 128, 92, FAKE, None, None, None) == BAD_SHAPE
    assert p(FAKE, FAKE, 1, 4, 128, -1, FAKE, None, None, None) == BAD_RANGE
    assert p(FAKE, FAKE, 1, 4, 128, 513, FAKE, None, None, None) == BAD_RANGE
    assert p(FAKE, FAKE, 1, 4, 128, 92, FAKE, P(4), None, None) == ALIGN         # theta 8 B


def test_append_plan_validation(L):
    """fathom_append_plan checks both calls' arguments: each failure of
    fathom_encode's or fathom_plan's checks, and the same codes."""
    a = L.fathom_append_plan
    enc = (FAKE, 1, 4096, 128, 64, 0, FAKE, FAKE, None)
    pl = (FAKE, FAKE, 4, 92, FAKE, None, None, None)

    def call(e=enc, p=pl):
        return a(*e, *p)
    assert call() != NULL_ARG
    assert call(e=(None,) + enc[1:]) == NULL_ARG                                # k
    assert call(e=enc[:6] + (None,) + enc[7:]) == NULL_ARG                      # planes
    assert call(e=enc[:7] + (None,) + enc[8:]) == NULL_ARG                      # scales
    assert call(p=(None,) + pl[1:]) == NULL_ARG                                 # q
    assert call(p=pl[:1] + (None,) + pl[2:]) == NULL_ARG                        # var
    assert call(p=pl[:4] + (None,) + pl[5:]) == NULL_ARG                        # depths
    assert call(e=enc[:3] + (64,) + enc[4:]) == BAD_SHAPE                       # d != 128
    assert call(e=(FAKE, 0) + enc[2:]) == BAD_SHAPE                             # groups
    assert call(e=(FAKE, 1, 4000) + enc[3:]) == BAD_SHAPE                       # n % 64
    assert call(e=enc[:4] + (63,) + enc[5:]) == BAD_SHAPE                       # capacity
    assert call(e=enc[:4] + (70, 7) + enc[6:]) == BAD_SHAPE                     # offset + nb
    assert call(p=(FAKE, FAKE, 0) + pl[3:]) == BAD_SHAPE                        # G
    assert call(p=(FAKE, FAKE, 9) + pl[3:]) == BAD_SHAPE
    assert call(p=(FAKE, FAKE, 4, -1) + pl[4:]) == BAD_RANGE                    # budget
    assert call(p=(FAKE, FAKE, 4, 513) + pl[4:]) == BAD_RANGE
    assert call(e=(P(8),) + enc[1:]) == ALIGN                                   # k 16 B
    assert call(e=enc[:8] + (P(2),)) == ALIGN                                   # flag 4 B
    assert call(p=pl[:5] + (P(4), None, None)) == ALIGN                         # theta 8 B


def test_plan_fixed_validation(L):
    p = L.fathom_plan_fixed
    L.fathom_plan_fixed.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, P, P]
    UNIFORM, SPARQ, TOPSTAT = 1, 2, 3
    assert p(FAKE, None, 1, 4, 128, UNIFORM, 2, None, None) == NULL_ARG
    assert p(None, FAKE, 1, 4, 128, SPARQ, 16, FAKE, None) == NULL_ARG
    assert p(FAKE, None, 1, 4, 128, TOPSTAT, 16, FAKE, None) == NULL_ARG
    assert p(FAKE, None, 1, 4, 100, SPARQ, 16, FAKE, None) == BAD_SHAPE
    assert p(FAKE, None, 1, 9, 128, SPARQ, 16, FAKE, None) == BAD_SHAPE
    assert p(FAKE, None, 0, 4, 128, SPARQ, 16, FAKE, None) == BAD_SHAPE
    assert p(None, None, 1, 4, 128, UNIFORM, 5, FAKE, None) == BAD_RANGE
    assert p(None, None, 1, 4, 128, UNIFORM, -1, FAKE, None) == BAD_RANGE
    assert p(FAKE, None, 1, 4, 128, SPARQ, 129, FAKE, None) == BAD_RANGE
    assert p(FAKE, None, 1, 4, 128, 7, 1, FAKE, None) == BAD_RANGE
    assert p(P(2), None, 1, 4, 128, SPARQ, 16, FAKE, None) == ALIGN
    assert p(None, None, 1, 4, 128, UNIFORM, 2, FAKE, None) == NO_DEVICE
    assert p(FAKE, None, 1, 4, 128, SPARQ, 16, FAKE, None) == NO_DEVICE


def test_scan_topk_validation(L):
    L.fathom_scan_topk.argtypes = [P, P, ctypes.c_int64, P, P, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, P,
                                   ctypes.c_size_t, P]
    L.fathom_scan_topk_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                                   ctypes.c_int32]
    L.fathom_scan_topk_workspace_bytes.restype = ctypes.c_size_t
    need = L.fathom_scan_topk_workspace_bytes(2, 4, 1 << 17, 256)
    assert need >= L.fathom_topk_workspace_bytes(8, 1 << 17, 256) > 0
    assert need >= 8 * (1 << 17) * 4          # room for every row's scores
    assert L.fathom_scan_topk_workspace_bytes(2, 4, 1 << 17, 0) == 0
    assert L.fathom_scan_topk_workspace_bytes(2, 9, 1 << 17, 1) == 0
    f = L.fathom_scan_topk
    args = [FAKE, FAKE, 2048, FAKE, FAKE, 2, 4, 128, 1 << 17, 256, FAKE, FAKE, FAKE, need, None]
    for i in (0, 1, 3, 4, 11, 12):
        a = list(args)
        a[i] = None
        assert f(*a) == NULL_ARG, i
    a = list(args)
    a[10] = None                               # no score buffer: a valid call
    assert f(*a) in (NO_DEVICE, OK) or _gpu_visible()
    for i, v in ((6, 9), (7, 64), (8, 1000), (2, 100)):
        a = list(args)
        a[i] = v
        assert f(*a) == BAD_SHAPE, (i, v)
    a = list(args)
    a[9] = 0
    assert f(*a) == BAD_RANGE
    a = list(args)
    a[12] = P((1 << 20) + 64)
    assert f(*a) == ALIGN
    a = list(args)
    a[13] = need - 1
    assert f(*a) == WORKSPACE
    assert f(*args) == NO_DEVICE


def test_gather_validation(L):
    L.fathom_gather.argtypes = [P, P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int64, P, P, P]
    g = L.fathom_gather
    args = [FAKE, FAKE, 64, FAKE, 2, 128, 4096, FAKE, FAKE, None]
    for i in (0, 1, 3, 7, 8):
        a = list(args)
        a[i] = None
        assert g(*a) == NULL_ARG, i
    for i, v in ((2, 60), (2, 63), (5, 64), (4, 0), (6, 100)):
        a = list(args)
        a[i] = v
        assert g(*a) == BAD_SHAPE, (i, v)
    a = list(args)
    a[0] = P((1 << 20) + 8)
    assert g(*a) == ALIGN
    assert g(*args) == NO_DEVICE


def test_klt_validation(L):
    def fit_bytes(groups, P):     # mean partials, product partials (one per chunk), covariance
        return groups * (P * 128 + P * 128 * 128 + 128 * 128) * 8
    assert L.fathom_klt_fit_workspace_bytes(8, 1 << 20, 128) == fit_bytes(8, 64)
    assert L.fathom_klt_fit_workspace_bytes(128, 1 << 17, 128) == fit_bytes(128, 4)
    assert L.fathom_klt_fit_workspace_bytes(1, 64, 128) == fit_bytes(1, 1)
    assert L.fathom_klt_fit_workspace_bytes(1, 100, 128) == 0
    need = L.fathom_klt_fit_workspace_bytes(2, 4096, 128)
    f = L.fathom_klt_fit
    args = [FAKE, 2, 4096, 128, FAKE, FAKE, FAKE, FAKE, need, None]
    for i in (0, 4, 5, 6, 7):
        a = list(args)
        a[i] = None
        assert f(*a) == NULL_ARG, i
    for i, v in ((1, 0), (2, 100), (2, 0), (3, 64)):
        a = list(args)
        a[i] = v
        assert f(*a) == BAD_SHAPE, (i, v)
    a = list(args)
    a[7] = P((1 << 20) + 16)
    assert f(*a) == ALIGN
    a = list(args)
    a[8] = need - 1
    assert f(*a) == WORKSPACE
    assert f(*args) == NO_DEVICE

    r = L.fathom_klt_rotate_keys
    args = [FAKE, FAKE, FAKE, 2, 4096, 128, FAKE, None]
    for i in (0, 1, 2, 6):
        a = list(args)
        a[i] = None
        assert r(*a) == NULL_ARG, i
    for i, v in ((3, 0), (4, 96), (5, 127)):
        a = list(args)
        a[i] = v
        assert r(*a) == BAD_SHAPE, (i, v)
    for i in (0, 2, 6):
        a = list(args)
        a[i] = P((1 << 20) + 4)
        assert r(*a) == ALIGN, i
    assert r(*args) == NO_DEVICE

    rq = L.fathom_klt_rotate_queries
    args = [FAKE, FAKE, 2, 4, 128, FAKE, None]
    for i in (0, 1, 5):
        a = list(args)
        a[i] = None
        assert rq(*a) == NULL_ARG, i
    for i, v in ((2, 0), (3, 0), (3, 9), (4, 64)):
        a = list(args)
        a[i] = v
        assert rq(*a) == BAD_SHAPE, (i, v)
    assert rq(*args) == NO_DEVICE


def test_scan_validation(L):
    s = L.fathom_scan
    args = [FAKE, FAKE, 64, FAKE, FAKE, 1, 4, 128, 4096, FAKE, None]
    for i in (0, 1, 3, 4, 9):
        a = list(args)
        a[i] = None
        assert s(*a) == NULL_ARG
    a = list(args); a[2] = 63
    assert s(*a) == BAD_SHAPE                                                     # nb_store < n/64
    a = list(args); a[6] = 9
    assert s(*a) == BAD_SHAPE
    a = list(args); a[7] = 256
    assert s(*a) == BAD_SHAPE
    a = list(args); a[8] = 4095
    assert s(*a) == BAD_SHAPE
    a = list(args); a[8] = 0
    assert s(*a) == BAD_SHAPE
    a = list(args); a[5] = 0
    assert s(*a) == BAD_SHAPE
    a = list(args); a[0] = P(4)
    assert s(*a) == ALIGN


def test_scan_timed_validation(L):
    s = L.fathom_scan_timed
    args = [FAKE, FAKE, 64, FAKE, FAKE, 1, 4, 128, 4096, FAKE, FAKE, FAKE, None]
    for i in (0, 1, 3, 4, 9, 10, 11):
        a = list(args)
        a[i] = None
        assert s(*a) == NULL_ARG
    a = list(args); a[2] = 63
    assert s(*a) == BAD_SHAPE
    a = list(args); a[6] = 0
    assert s(*a) == BAD_SHAPE
    a = list(args); a[8] = 4095
    assert s(*a) == BAD_SHAPE
    a = list(args); a[0] = P(4)
    assert s(*a) == ALIGN


def test_topk_validation(L):
    t = L.fathom_topk
    need = L.fathom_topk_workspace_bytes(4, 1000, 10)
    assert need > 0 and need % 256 == 0
    assert t(None, 4, 1000, 10, FAKE, FAKE, need, None) == NULL_ARG
    assert t(FAKE, 4, 1000, 10, FAKE, None, need, None) == NULL_ARG
    assert t(FAKE, 0, 1000, 10, FAKE, FAKE, need, None) == BAD_SHAPE
    assert t(FAKE, 4, 0, 1, FAKE, FAKE, need, None) == BAD_SHAPE
    assert t(FAKE, 4, 1000, 0, FAKE, FAKE, need, None) == BAD_RANGE
    assert t(FAKE, 4, 1000, 1001, FAKE, FAKE, need, None) == BAD_RANGE
    assert t(FAKE, 4, 1000, 10, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert t(FAKE, 4, 1000, 10, FAKE, P((1 << 20) + 128), need, None) == ALIGN
    assert L.fathom_topk_workspace_bytes(4, 1000, 1001) == 0
    assert L.fathom_topk_workspace_bytes(8, 1 << 20, 4096) >= L.fathom_topk_workspace_bytes(4, 1 << 20, 4096)


def test_topk_noalloc_validation(L):
    """The no-allocation top-k checks its arguments like fathom_topk and
    rejects calls whose workspace would exceed its fixed scratch."""
    t = L.fathom_topk_noalloc
    cap = L.fathom_topk_noalloc_max_bytes()
    assert cap == 64 << 20
    assert t(None, 4, 1000, 10, FAKE, None) == NULL_ARG
    assert t(FAKE, 4, 1000, 10, None, None) == NULL_ARG
    assert t(FAKE, 0, 1000, 10, FAKE, None) == BAD_SHAPE
    assert t(FAKE, 4, 1000, 0, FAKE, None) == BAD_RANGE
    assert t(FAKE, 4, 1000, 10, P((1 << 20) + 2), None) == ALIGN
    # 32 rows of 2^20 keys fit; 512 rows of 131,072 keys (76 MB) do not
    assert L.fathom_topk_workspace_bytes(32, 1 << 20, 4096) <= cap
    assert L.fathom_topk_workspace_bytes(512, 131072, 1024) > cap
    assert t(FAKE, 512, 131072, 1024, FAKE, None) == -9


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device status; a GPU is visible")
def test_valid_calls_report_no_device(L):
    assert L.fathom_scan(FAKE, FAKE, 64, FAKE, FAKE, 1, 4, 128, 4096, FAKE, None) == NO_DEVICE
    need = L.fathom_topk_workspace_bytes(4, 1000, 10)
    assert L.fathom_topk(FAKE, 4, 1000, 10, FAKE, FAKE, need, None) == NO_DEVICE
    assert L.fathom_topk_noalloc(FAKE, 4, 1000, 10, FAKE, None) == NO_DEVICE
    assert L.fathom_plan(FAKE, FAKE, 1, 4, 128, 92, FAKE, None, None, None) == NO_DEVICE
    assert L.fathom_encode(FAKE, 1, 4096, 128, 64, 0, FAKE, FAKE, None, None) == NO_DEVICE
    assert L.fathom_append_plan(FAKE, 1, 4096, 128, 64, 0, FAKE, FAKE, None, FAKE, FAKE, 4, 92,
                                FAKE, None, None, None) == NO_DEVICE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding has no fallback: a missing library raises on first use."""
    import importlib
    import sparse_top_kv_fathom_amd._binding as b
    monkeypatch.setattr(b, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(ImportError):
        b.lib()
    importlib.reload(b)


def test_cut_hooks_reject_bad_arguments(L):
    """fathom_test_cut_hooks checks its arguments on the host (no GPU call)."""
    for publish, spin in ((2, 16), (-1, 16), (1, 0), (1, 16385), (0, -3)):
        assert L.fathom_test_cut_hooks(publish, spin) == BAD_RANGE
    assert L.fathom_test_cut_hooks(1, 2048) == OK
