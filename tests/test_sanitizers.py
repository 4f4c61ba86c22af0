"""The fp64 oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

- The oracle (C, gcc) is built with both sanitizers together with a driver
  (tests/sanitize/oracle_driver.c) that calls every entry point on seeded
  inputs in buffers of exactly the documented sizes.
- The library's host code (hsv_api.cpp: descriptor checks, planning,
  workspace sizes, argument checks) is rebuilt with both sanitizers on the
  host side only and linked with the normal objects of the other sources;
  tests/sanitize/host_driver.py then fuzzes descriptors and calls every entry
  point with arguments it must reject before any device work, in a process
  that has clang's sanitizer runtime preloaded.

Each driver exits non-zero on a sanitizer report or a wrong status.
"""

import glob
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
PKG = os.path.join(ROOT, "long_context_tree_verify_amd")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", "-I", ORACLE, os.path.join(ORACLE, "oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = _run([exe], env=env)
    assert "all cases passed" in r.stdout


def _build_lib_module():
    spec = importlib.util.spec_from_file_location("hsv_build_lib", os.path.join(PKG, "build_lib.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_library_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not runtimes:
        pytest.skip("hipcc or clang's sanitizer runtime not found")
    bl = _build_lib_module()
    others = [s for s in bl.SOURCES if s != "hsv_api.cpp"]
    objs = [os.path.join(bl.BUILD, s + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs):
        bl.build()
    api_obj = str(tmp_path / "hsv_api.o")
    lib = str(tmp_path / "libhsv_sanitized.so")
    # sanitizers on the host side only: each -fsanitize= behind -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    _run([hipcc, f"--offload-arch={bl.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
          f"-I{bl.INCLUDE}", f"-I{bl.CSRC}", *host_san,
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(bl.CSRC, "hsv_api.cpp"), "-o", api_obj])
    _run([hipcc, f"--offload-arch={bl.ARCH}", "-shared", "-fPIC", *host_san, "-o", lib, api_obj,
          *objs])
    env = dict(os.environ, LD_PRELOAD=runtimes[0], ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([sys.executable, os.path.join(HERE, "host_driver.py"), lib], env=env)
    assert "all cases passed" in r.stdout
