"""The C ABI from a C program: tests/c_abi/host_check.c compiled as C11
(gcc) and as C++17 (g++), with warnings as errors, against include/hsv.h
and linked with libhsv.so; each build runs the host-side checks (no GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "host_check.c")
LIBDIR = os.path.join(ROOT, "long_context_tree_verify_amd")


@pytest.fixture(scope="module")
def libhsv():
    if not os.path.exists(os.path.join(LIBDIR, "libhsv.so")):
        import importlib.util
        spec = importlib.util.spec_from_file_location("hsv_build_lib",
                                                      os.path.join(LIBDIR, "build_lib.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return LIBDIR


@pytest.mark.parametrize("compiler,std,lang", [("gcc", "c11", "c"), ("g++", "c++17", "c++")])
def test_header_and_library_from_c(libhsv, tmp_path, compiler, std, lang):
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / "host_check")
    cmd = [cc, "-x", lang, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include", SRC, "-x", "none",
           f"-L{libhsv}", "-lhsv", f"-Wl,-rpath,{libhsv}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
