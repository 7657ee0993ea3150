"""Build libfathom.so (gfx950) in the package directory with hipcc.

Every kernel source is compiled for gfx950 only, with floating-point
contraction off (the scan's fp32 order is part of its contract) and the
packed-fp32 instructions disabled.  Run ``python -m sparse_top_kv_fathom_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfathom.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["api.hip", "encode.hip", "plan.hip", "scan.hip", "topk.hip", "gather.hip", "klt.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfathom.so)")


def _compile(src: str) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libfathom.so; returns its path."""
    with cf.ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def asm(src: str, out: str) -> None:
    """Device assembly of one source (for inspecting the generated gfx950 code)."""
    cmd = [hipcc(), *HIPCC_FLAGS, "--offload-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
