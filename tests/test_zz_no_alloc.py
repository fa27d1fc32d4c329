"""fp8_quantize_no_workspace, the variant of fp8_quantize whose per-tensor
partial maxima live in the library's static device scratch instead of a
caller workspace, called through the C ABI and compared bit for bit with
fp8_quantize given a workspace: two calls in a row on one stream, the
second on a smaller input, so the second reuses what the first left in the
scratch.  Per-tensor scaling from the amax on the streamed path (a tensor
larger than the infinity cache, 8192 partials) and on the folded path (a
small ragged one), both formats, BF16 and FP32 input; block granularities
and given scales, which need no scratch, pass straight through."""
import ctypes

import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _entry():
    L = gs.lib()
    f = L.fp8_quantize_no_workspace
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [P, I, I64, I64, I, I, I, P, P, P, P]
    f.restype = ctypes.c_int32
    return f


def _no_ws(x, fmt, gran, mode, codes, scales, nonfinite):
    """One call straight through the C ABI (ctypes), no binding checks."""
    rows, cols = x.shape
    dt = gs.GS_BF16 if x.dtype == torch.bfloat16 else gs.GS_F32
    st = _entry()(x.data_ptr(), dt, rows, cols, fmt, gran, mode, codes.data_ptr(),
                  scales.data_ptr(), nonfinite.data_ptr(),
                  torch.cuda.current_stream().cuda_stream)
    assert st == gs.GS_OK, gs.status_string(st)


def _input(rng, rows, cols, dtype, dev):
    x = torch.from_numpy(rng.standard_normal((rows, cols), dtype=np.float32)).to(dev)
    x[rows // 3, cols // 2] = 700.0                      # an outlier sets the amax
    x[rows - 1, cols - 1] = float("nan")                 # ignored by the amax, flagged
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_no_workspace_matches_fp8_quantize(dev, dtype):
    rng = np.random.default_rng(1707)
    big = (16384, 8192) if dtype == torch.bfloat16 else (8192, 8192)   # 256 MiB: 8192 partials
    cases = [(big, gs.FP8_PER_TENSOR, gs.FP8_SCALE_FROM_AMAX),
             ((1000, 777), gs.FP8_PER_TENSOR, gs.FP8_SCALE_FROM_AMAX),  # folded, ragged
             ((512, 1024), gs.FP8_BLOCK_1x128, gs.FP8_SCALE_FROM_AMAX),
             ((256, 384), gs.FP8_BLOCK_128x128, gs.FP8_SCALE_FROM_AMAX),
             ((64, 96), gs.FP8_PER_TENSOR, gs.FP8_SCALE_GIVEN)]
    for fmt in (gs.FP8_E4M3, gs.FP8_E5M2):
        xs = [_input(rng, r, c, dtype, dev) for (r, c), _, _ in cases]
        outs = []
        for x, (shape, gran, mode) in zip(xs, cases):      # all enqueued back to back
            codes = torch.full(shape, 0xAA, dtype=torch.uint8, device=dev)
            if mode == gs.FP8_SCALE_GIVEN:
                scales = torch.tensor([0.75], dtype=torch.float32, device=dev)
            else:
                scales = torch.full(gs.scale_shape(*shape, gran), -1.0, dtype=torch.float32,
                                    device=dev)
            nf = torch.zeros(1, dtype=torch.int32, device=dev)
            _no_ws(x, fmt, gran, mode, codes, scales, nf)
            outs.append((codes, scales, nf))
        for x, (shape, gran, mode), (codes, scales, nf) in zip(xs, cases, outs):
            ref_scales = scales.clone() if mode == gs.FP8_SCALE_GIVEN else None
            nf_ref = torch.zeros(1, dtype=torch.int32, device=dev)
            rc, rs = gs.fp8_quantize(x, fmt, gran, mode, scales=ref_scales, nonfinite=nf_ref)
            torch.cuda.synchronize()
            tag = (str(dtype), fmt, shape, gran, mode)
            assert torch.equal(codes, rc), tag
            assert torch.equal(scales.view(torch.int32), rs.view(torch.int32)), tag
            assert int(nf.item()) == int(nf_ref.item()) == 1, tag


def test_binding_wrapper_matches(dev):
    """The binding's wrapper of the same entry point, on a folded per-tensor
    case, against fp8_quantize."""
    x = _input(np.random.default_rng(1708), 777, 1000, torch.bfloat16, dev)
    codes = torch.empty((777, 1000), dtype=torch.uint8, device=dev)
    scales = torch.empty(1, dtype=torch.float32, device=dev)
    gs.fp8_quantize_no_workspace(x, gs.FP8_E5M2, gs.FP8_PER_TENSOR, codes, scales)
    rc, rs = gs.fp8_quantize(x, gs.FP8_E5M2, gs.FP8_PER_TENSOR)
    torch.cuda.synchronize()
    assert torch.equal(codes, rc) and torch.equal(scales.view(torch.int32), rs.view(torch.int32))


def test_no_workspace_argument_errors(dev):
    """Argument errors come back before any launch, as for fp8_quantize."""
    f = _entry()
    x = torch.zeros((128, 128), dtype=torch.bfloat16, device=dev)
    c = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    s = torch.zeros(1, dtype=torch.float32, device=dev)
    assert f(x.data_ptr(), 7, 128, 128, 0, 0, 0, c.data_ptr(), s.data_ptr(), None, None) == -4
    assert f(x.data_ptr(), gs.GS_BF16, 128, 100, 0, 1, 0, c.data_ptr(), s.data_ptr(), None,
             None) == -3
    assert f(None, gs.GS_BF16, 128, 128, 0, 0, 0, c.data_ptr(), s.data_ptr(), None, None) == -1
    assert f(x.data_ptr() + 2, gs.GS_BF16, 8, 8, 0, 0, 0, c.data_ptr(), s.data_ptr(), None,
             None) == -6
