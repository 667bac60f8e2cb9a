"""The C ABI layer under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

api.cpp is rebuilt with -fsanitize=address,undefined and linked with the regular
kernels' objects (activation_sparse_gemv_amd/sanitize_build.py); test_abi.py then
runs in a child process with the sanitizer runtime preloaded and the sanitized
library loaded in place of the regular one.  Any sanitizer report fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    from activation_sparse_gemv_amd import build as B
    from activation_sparse_gemv_amd import sanitize_build as S
    if not os.path.exists(B.LIB) or not os.path.isdir(B.BUILD):
        pytest.skip("the regular library is not built (python -m activation_sparse_gemv_amd.build)")
    lib = S.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=S.asan_runtime(), ACTSPARSE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child loads the sanitized library (its instrumentation symbols are present)
    probe = ("import ctypes; from activation_sparse_gemv_amd import _lib as L; L.load(); "
             "h = ctypes.CDLL(L.LIB_PATH); print(L.LIB_PATH, hasattr(h, '__asan_report_load4'))")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == [lib, "True"], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
