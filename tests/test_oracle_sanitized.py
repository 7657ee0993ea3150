"""The oracle's CPU pins again, with fathom_oracle.c built under
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host code only): an
out-of-bounds access, use of freed memory or undefined integer behaviour in
the oracle makes this test fail instead of silently shifting its results.

The pins run in a child interpreter with the sanitizer runtimes preloaded
(the interpreter itself is not instrumented) and FATHOM_ORACLE_LIB pointing
the oracle at the instrumented build."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_encode.py", "tests/test_oracle_plan.py",
             "tests/test_oracle_scan.py", "tests/test_oracle_topk.py",
             "tests/test_oracle_klt.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not available")
    lib = str(tmp_path / "libfathom_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-o", lib, os.path.join(ROOT, "oracle", "fathom_oracle.c"), "-lm"],
                   check=True)
    env = dict(os.environ,
               LD_PRELOAD=asan + ":" + ubsan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               FATHOM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=840)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stderr.lower(), tail
