"""Build libgsfp8.so (the HIP library behind include/gs.h) for gfx950, and
libgsceil.so (the streaming kernels the benchmark measures its ceilings
with; not part of the library).

    python -m loss_scaling_fp8_amd.build

Each csrc/*.hip file is compiled to an object in parallel, then linked into
loss_scaling_fp8_amd/libgsfp8.so; ceilings/*.hip are linked into
loss_scaling_fp8_amd/libgsceil.so.  Packed FP32 instructions are disabled for
all device code (-Xclang -target-feature -Xclang -packed-fp32-ops; the host
pass warns that it does not know the feature, which is harmless).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgsfp8.so")
CEIL_DIR = os.path.join(PKG, "ceilings")
CEIL_LIB = os.path.join(PKG, "libgsceil.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def ceiling_sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CEIL_DIR, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build_variant(lib: str, defines: list[str]) -> str:
    """The library built with extra preprocessor definitions (for example the
    tiny grid caps of a test build), linked to `lib`; objects go to a
    directory of their own beside it."""
    obj_dir = os.path.join(os.path.dirname(lib), "_obj_" + os.path.basename(lib))
    os.makedirs(obj_dir, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *CXXFLAGS, *defines, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
        return obj

    srcs = sources()
    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, srcs))
    _link(objs, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link both shared libraries (always)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs, csrcs = sources(), ceiling_sources()
    with ThreadPoolExecutor(min(len(srcs) + len(csrcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, srcs + csrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], CEIL_LIB)
    if verbose:
        print("built", LIB, "and", CEIL_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
