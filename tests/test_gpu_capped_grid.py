"""GPU parity of the grid-stride paths.  Every launch caps its grid (2^20
workgroups for quantize / dequantize, 2^22 for the unscale, the partial
slots for per-tensor and delayed scaling) and strides past the cap, which in
the real library happens only for tensors of several 10^9 elements.  Here
the same sources built with caps of 3 and 5 workgroups
(tests/c/_build/libgsfp8_capped_grid.so, built by __graft_entry__.build())
run the seeded random cases of test_gpu_random.py and the delayed-scaling
sequences of test_gpu_delayed.py, plus a per-tensor and a plain unscale
case, each against the oracle bit for bit: every kernel then loops over many
grid strides."""
import os

import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import test_gpu_delayed as delayed_cases
import test_gpu_random as random_cases

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAPPED = os.path.join(ROOT, "tests", "c", "_build", "libgsfp8_capped_grid.so")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


@pytest.fixture
def capped():
    """The binding's calls go to the capped-grid library for one test."""
    assert os.path.exists(CAPPED), "%s is not built (run __graft_entry__.build())" % CAPPED
    old_path, old_lib = gs.LIB_PATH, gs._lib
    gs.LIB_PATH, gs._lib = CAPPED, None
    try:
        yield gs.lib()
    finally:
        gs.LIB_PATH, gs._lib = old_path, old_lib


def test_the_capped_library_is_the_one_called(capped):
    assert gs.lib() is capped and gs.LIB_PATH == CAPPED


@pytest.mark.parametrize("seed", range(4))
def test_random_quantize_cases_strided(dev, capped, seed):
    random_cases.test_random_quantize_cases(dev, seed)


@pytest.mark.parametrize("seed", range(3))
def test_random_unscale_sumsq_lists_strided(dev, capped, seed):
    random_cases.test_random_unscale_sumsq_lists(dev, seed)


@pytest.mark.parametrize("fmt,dtype,hlen", [(gs.FP8_E4M3, "bf16", 4), (gs.FP8_E5M2, "f32", 16),
                                            (gs.FP8_E4M3, "f32", 1)])
def test_delayed_sequences_strided(dev, capped, fmt, dtype, hlen):
    delayed_cases.test_delayed_sequence_matches_oracle(fmt, dtype, hlen, dev)


def test_per_tensor_and_plain_unscale_strided(dev, capped):
    """Per-tensor scaling from the amax on 1.5M elements (3 partial maxima,
    each cast workgroup folds them; about 500 strides per workgroup), and
    the plain unscale over a 40-tensor list (about 50 chunks per
    workgroup)."""
    rng = np.random.default_rng(31)
    for fmt, dtype in ((gs.FP8_E4M3, "bf16"), (gs.FP8_E5M2, "f32")):
        xh = np.ascontiguousarray(random_cases._data(rng, 1024, 1536, dtype))
        x = random_cases._to_dev(xh, dev)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        codes, sc = gs.fp8_quantize(x, fmt, gs.FP8_PER_TENSOR, nonfinite=nf)
        deq = gs.fp8_dequantize(codes, fmt, gs.FP8_PER_TENSOR, sc)
        rc, rs, rnf = oracle.quantize(xh, fmt, gs.FP8_PER_TENSOR)
        rd = oracle.dequantize(rc, fmt, gs.FP8_PER_TENSOR, rs)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc), (fmt, dtype)
        assert random_cases._u32(sc)[0] == rs.view(np.uint32)[0], (fmt, dtype)
        assert np.array_equal(random_cases._u32(deq), rd.reshape(-1).view(np.uint32)), (fmt, dtype)
        assert int(nf.item()) == rnf == 1, (fmt, dtype)
    host = [rng.integers(0, 0x10000, size=int(n), dtype=np.uint32).astype(np.uint16)
            for n in rng.integers(1, 12000, 40)]
    grads = [torch.from_numpy(h.view(np.int16)).view(torch.float16).to(dev) for h in host]
    outs = [torch.empty(h.size, dtype=torch.float32, device=dev) for h in host]
    S = torch.tensor([1024.0], dtype=torch.float32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    gs.gs_unscale_check(grads, outs, S, found)
    ref, rflag = oracle.unscale_check(host, 1024.0)
    torch.cuda.synchronize()
    for t, (o, r) in enumerate(zip(outs, ref)):
        assert np.array_equal(random_cases._u32(o), r.view(np.uint32)), t
    assert int(found.item()) == rflag


def test_per_tensor_streaming_path_strided(dev, capped):
    """A tensor larger than the infinity cache (8192x12800 BF16, 210 MB)
    takes the other per-tensor path: the streaming partial-max pass, the
    one-workgroup finalize, then the cast; with the caps, 3 workgroups each
    stride over all of it."""
    rng = np.random.default_rng(37)
    rows, cols = 8192, 12800
    assert rows * cols * 2 > 192 << 20
    xf = rng.standard_normal((rows, cols), dtype=np.float32)
    xf.reshape(-1)[rng.integers(0, xf.size, 1000)] *= 1e4
    xf.reshape(-1)[rng.integers(0, xf.size, 10)] = np.nan
    xh = (xf.view(np.uint32) >> 16).astype(np.uint16)           # BF16 by truncation
    del xf
    x = random_cases._to_dev(xh, dev)
    for fmt in (gs.FP8_E4M3, gs.FP8_E5M2):
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        codes, sc = gs.fp8_quantize(x, fmt, gs.FP8_PER_TENSOR, nonfinite=nf)
        rc, rs, rnf = oracle.quantize(xh, fmt, gs.FP8_PER_TENSOR)
        torch.cuda.synchronize()
        assert random_cases._u32(sc)[0] == rs.view(np.uint32)[0], fmt
        assert np.array_equal(codes.cpu().numpy(), rc), fmt
        assert int(nf.item()) == rnf == 1, fmt
