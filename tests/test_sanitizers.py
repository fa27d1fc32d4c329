"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The oracle: oracle/oracle.c and the driver tests/c/oracle_sanitize.c
  built together by gcc with -fsanitize=address,undefined
  -fno-sanitize-recover=all; the driver calls every oracle entry point on
  exactly sized heap buffers.
* The library's host code (argument checks, the chunk-descriptor builder,
  status strings): libgsfp8's HIP sources rebuilt with the sanitizers on the
  host pass only, and tests/c/abi_host.c run against that build with clang's
  runtime.  Device code is built as usual; nothing here touches a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", *SAN,
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
          "-o", exe, "-lm"])
    r = _run([exe], timeout=300)
    assert "0 failure(s)" in r.stdout and "done" in r.stdout


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs ROCm")
def test_library_host_code_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "loss_scaling_fp8_amd", "csrc")
    srcs = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    host_san = []
    for f in SAN:                         # the host pass only: -Xarch_host before each flag
        host_san += ["-Xarch_host", f]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san]
    objs = []
    procs = []
    for f in srcs:
        o = str(tmp_path / (f + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(csrc, f), "-o", o],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-3000:]
    lib = str(tmp_path / "libgsfp8_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
          "-o", lib, *objs])
    exe = str(tmp_path / "abi_host_san")
    _run([CLANG, "-std=c99", "-O1", "-g", *SAN, "-I" + os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, lib,
          "-Wl,-rpath," + str(tmp_path)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = _run([exe], timeout=120, env=env)
    assert "0 failure(s)" in r.stdout
