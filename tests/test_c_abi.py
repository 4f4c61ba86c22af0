"""The C ABI from a C program: tests/c_abi/host_check.c compiled as C11
(gcc) and as C++17 (g++), with warnings as errors, against include/hsv.h
and linked with libhsv.so; each build runs the host-side checks (no GPU).
On the GPU, tests/c_abi/gpu_check.c (C11, HIP runtime API only) runs
hsv_verify_attn on device buffers, with the parent array and with the
bitmask hsv_tree_ancestor_mask builds, against the fp64 oracle."""

import os
import shutil
import subprocess

import numpy as np
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


def _gpu_check_exe(libdir, tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "gpu_check")
    cmd = [cc, "-x", "c", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi", "gpu_check.c"), "-x", "none", f"-L{libdir}",
           "-lhsv", "-L/opt/rocm/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{libdir}",
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _write_case(path, inp, o_ref, l_ref):
    B, N, Hq, D = inp.q.shape
    _, Hkv, cap, _ = inp.k.shape
    head = np.array([B, N, Hq, Hkv, D, cap, 1 if inp.is_bf16 else 0, int(inp.ctx_lens.max()),
                     0x48535643], "<i4")
    with open(path, "wb") as f:
        for a in (head, inp.q, inp.k, inp.v):
            f.write(np.ascontiguousarray(a).tobytes())
        f.write(np.ascontiguousarray(inp.ctx_lens, "<i4").tobytes())
        f.write(np.ascontiguousarray(inp.parent, "<i4").tobytes())
        f.write(np.ascontiguousarray(o_ref, "<f8").tobytes())
        f.write(np.ascontiguousarray(l_ref, "<f8").tobytes())


@pytest.mark.gpu
@pytest.mark.parametrize("name,over", [
    ("tiny_tree", dict(batch=2, ctx=(0, 256))),                 # fp32 kernel
    ("tree32k", dict(ctx=(1500, 1500))),                        # 256-row DMA kernel
    ("chain_b16", dict(batch=3, ctx=(300, 900))),               # small-group kernel
    ("tree32k", dict(n_draft=100, max_depth=10, ctx=(700, 700))),  # two-word masks
])
def test_verify_from_c_on_gpu(libhsv, gpu, tmp_path, name, over):
    import oracle
    import synth
    from util import log
    exe = _gpu_check_exe(libhsv, tmp_path)
    inp = synth.make_inputs(name, seed=7400, **over)
    o_ref, l_ref = oracle.verify_attn(inp.q, inp.k, inp.v, inp.ctx_lens, parent=inp.parent,
                                      bf16=inp.is_bf16)
    path = str(tmp_path / "case.bin")
    _write_case(path, inp, o_ref, l_ref)
    log(f"C caller on the GPU: {name} {over}")
    r = subprocess.run([exe, path], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
