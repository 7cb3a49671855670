"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (``oracle/la_oracle.c``) is built with gcc and both sanitizers and
  run over every routine on small and ragged shapes (``oracle/sanity_main.c``).
* The library is rebuilt with its host code instrumented (the device code is
  compiled as usual, and never run here), and ``tests/abi_sanity.c`` drives the
  argument validation, workspace sizing, plan and diagnostic entry points of
  the C ABI through it: every call fails validation, so no GPU is needed.

Both builds go to ``_build/sanitize/``.  Sanitizers are never applied to GPU
code: on each hipcc line every ``-fsanitize=`` sits right after
``-Xarch_host``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "kernelized_transformer_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_sanity")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "la_oracle.c"), os.path.join(ROOT, "oracle", "sanity_main.c"), "-o", exe,
          "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle sanity: ok" in r.stdout


def test_abi_host_code_under_asan_ubsan():
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "lib", "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(OUT, "libla_sanitize.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib, *HOST_SAN])
    exe = os.path.join(OUT, "abi_sanity")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
          os.path.join(ROOT, "tests", "abi_sanity.c"), "-o", exe, lib, "-Wl,-rpath," + OUT,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    r = _run([exe], env=ENV)
    assert "abi sanity: ok" in r.stdout
