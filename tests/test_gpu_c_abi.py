"""The C ABI from a plain C program on the GPU: tests/c/_build/abi_gpu (built
by __graft_entry__.build() from tests/c/abi_gpu.c) allocates with hipMalloc,
calls every compute entry point of include/gs.h on a stream of its own, and
compares each result bit for bit with the C oracle linked beside it: the
unscale and the update over three steps (an Inf on the second), the exact
sum of squares, the hysteresis policy, quantize and FP32 / BF16 dequantize
at every granularity in both formats, the per-tensor quantize without a
workspace, MX blocks and three delayed-scaling
steps.  No Python, torch or ctypes between the caller and the library."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "_build", "abi_gpu")


def test_c_caller_on_the_gpu():
    assert os.path.exists(EXE), "tests/c/_build/abi_gpu is not built: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "0 failure(s)" in r.stdout
    assert r.stdout.count("ok  ") >= 30
