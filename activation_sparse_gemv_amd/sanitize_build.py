"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI layer.

    python -m activation_sparse_gemv_amd.sanitize_build

Compiles ``csrc/api.cpp`` (argument validation, plans, workspace carving, the
host-side computations) with ``-fsanitize=address,undefined`` and links it with
the kernels' objects of the regular build (``_build/``, built first if needed)
into ``_build_asan/libactsparse_asan.so``.  Only host code is instrumented; the
device code is the regular build's.  Load it with the sanitizer runtime preloaded
(``asan_runtime()``), e.g. ``LD_PRELOAD=<runtime> ACTSPARSE_LIB=<lib> pytest
tests/test_abi.py``: the ABI tests then run every validation path and host
computation under the sanitizers.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as B

LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang++")
OUT = os.path.join(B.ROOT, "_build_asan")
LIB = os.path.join(OUT, "libactsparse_asan.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm LLVM toolchain."""
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + LLVM)
    return hits[-1]


def build_sanitized() -> str:
    B.build(incremental=True)
    os.makedirs(OUT, exist_ok=True)
    api_obj = os.path.join(OUT, "api.cpp.o")
    src = os.path.join(B.CSRC, "api.cpp")
    compile_cmd = [CLANG, "-O1", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                   "-I", os.path.join(B.ROOT, "include"), *SAN, "-c", src, "-o", api_obj]
    r = subprocess.run(compile_cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile of api.cpp failed:\n{r.stdout}\n{r.stderr}")
    objs = [api_obj] + [o for o in sorted(glob.glob(os.path.join(B.BUILD, "*.o")))
                        if os.path.basename(o) != "api.cpp.o"]
    tmp = LIB + ".tmp"
    link_cmd = [CLANG, "-shared", "-fPIC", *SAN, "-shared-libasan", "-o", tmp, *objs,
                "-L/opt/rocm/lib", "-lamdhip64", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(link_cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
    sys.exit(0)
