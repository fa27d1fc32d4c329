"""Builds tests/c/_build/abi_gpu: tests/c/abi_gpu.c, a plain C11 caller of
libgsfp8 on the GPU, linked against the built library, the oracle's
oracle/_build/liboracle.so and the HIP runtime (run paths relative to the
binary, so the tree can move).  Needs both libraries built first.

    python tests/c/build_abi_gpu.py [OUT]
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out=None):
    out = out or os.path.join(HERE, "_build", "abi_gpu")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    rel = os.path.relpath(ROOT, os.path.dirname(out))
    rpath = ":".join(["$ORIGIN/" + rel + "/loss_scaling_fp8_amd", "$ORIGIN/" + rel + "/oracle/_build",
                      os.path.join(ROCM, "lib")])
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_gpu.c"), "-o", out,
           "-L" + os.path.join(ROOT, "loss_scaling_fp8_amd"), "-l:libgsfp8.so",
           "-L" + os.path.join(ROOT, "oracle", "_build"), "-l:liboracle.so",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + rpath]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else None))
