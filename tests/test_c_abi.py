"""The C ABI from C: tests/c/abi_host.c is compiled as strict C99 against
include/gs.h, linked against the built libgsfp8.so, and run (host-only
entry points and argument checks; no GPU needed); tests/c/abi_gpu.c, the C
caller the GPU tests run, is compiled and linked."""
import os
import shutil
import subprocess

import pytest

import loss_scaling_fp8_amd as gs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c99_caller(tmp_path):
    lib = gs.LIB_PATH
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    exe = str(tmp_path / "abi_host")
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
           "-o", exe, "-L" + libdir, "-l:" + os.path.basename(lib), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_gpu_caller_builds(tmp_path):
    """tests/c/abi_gpu.c (run by the GPU tests) compiles as strict C11
    against include/gs.h and links against the built library, the oracle
    and the HIP runtime; nothing is run here."""
    import runpy
    mod = runpy.run_path(os.path.join(ROOT, "tests", "c", "build_abi_gpu.py"))
    exe = mod["build"](str(tmp_path / "abi_gpu"))
    assert os.path.exists(exe)
