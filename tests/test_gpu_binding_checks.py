"""The Python binding's argument checks on GPU tensors: buffers too short for
what a kernel writes, wrong element types and non-contiguous views are
refused before anything is enqueued (the C ABI takes bare pointers and could
not see them), and the outputs are left untouched."""
import pytest
import torch

import loss_scaling_fp8_amd as gs

pytestmark = pytest.mark.gpu

E4M3, B1, B128, PT = gs.FP8_E4M3, gs.FP8_BLOCK_1x128, gs.FP8_BLOCK_128x128, gs.FP8_PER_TENSOR


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def test_short_output_buffers(dev):
    x = torch.ones(256, 256, dtype=torch.bfloat16, device=dev)
    codes = torch.full((256, 256), 7, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="scales holds"):
        gs.fp8_quantize(x, E4M3, B1, codes=codes, scales=torch.zeros(255, 2, device=dev))
    with pytest.raises(ValueError, match="codes holds"):
        gs.fp8_quantize(x, E4M3, B1, codes=codes[:255])
    with pytest.raises(ValueError, match="out holds"):
        gs.fp8_dequantize(codes, E4M3, B128, torch.ones(2, 2, device=dev),
                          out=torch.empty(256, 255, device=dev))
    with pytest.raises(ValueError, match="scales holds"):
        gs.fp8_dequantize_bf16(codes, E4M3, B128, torch.ones(3, device=dev))
    with pytest.raises(ValueError, match="scales holds"):
        gs.fp8_quantize_mx(x, E4M3, scales=torch.zeros(256, 7, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="workspace holds"):
        gs.fp8_quantize(x, E4M3, PT, workspace=torch.zeros(16, dtype=torch.uint8, device=dev))
    S = torch.ones(1, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    g = [torch.ones(5000, dtype=torch.float16, device=dev)]
    o = [torch.zeros(5000, device=dev)]
    with pytest.raises(ValueError, match="workspace holds"):
        gs.gs_unscale_check_sumsq(g, o, S, f, torch.zeros(2, dtype=torch.int64, device=dev),
                                  torch.zeros(1, dtype=torch.float64, device=dev),
                                  workspace=torch.zeros(8, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="sumsq holds"):
        gs.gs_unscale_check_sumsq(g, o, S, f, torch.zeros(1, dtype=torch.int64, device=dev),
                                  torch.zeros(1, dtype=torch.float64, device=dev))
    torch.cuda.synchronize()
    assert bool((codes == 7).all()) and bool((o[0] == 0).all()) and int(f.item()) == 0


def test_wrong_element_types(dev):
    S = torch.ones(1, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(TypeError, match="found_inf"):
        gs.gs_update_scale(S, f, torch.zeros(1, dtype=torch.int64, device=dev))
    with pytest.raises(TypeError, match="scale"):
        gs.gs_update_scale(torch.ones(1, dtype=torch.float64, device=dev), f, f)
    with pytest.raises(TypeError, match="skip_count"):
        gs.gs_update_scale(S, f, f, skip_count=torch.zeros(1, dtype=torch.int32, device=dev))
    with pytest.raises(TypeError, match="history_pos"):
        gs.fp8_quantize_delayed(torch.ones(4, 4, device=dev), E4M3, S,
                                torch.zeros(4, device=dev), torch.zeros(1, dtype=torch.int64, device=dev))
    codes = torch.zeros(128, 128, dtype=torch.uint8, device=dev)
    with pytest.raises(TypeError, match="out"):
        gs.fp8_dequantize_bf16(codes, E4M3, B128, torch.ones(1, device=dev),
                               out=torch.empty(128, 128, dtype=torch.float16, device=dev))
    torch.cuda.synchronize()
    assert float(S.item()) == 1.0 and int(f.item()) == 0


def test_non_contiguous_views(dev):
    x = torch.ones(256, 512, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        gs.fp8_quantize(x.t(), E4M3, B1)
    codes = torch.zeros(256, 512, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        gs.fp8_dequantize(codes[:, :256], E4M3, B1, torch.ones(256, 2, device=dev))
    g = torch.ones(100, dtype=torch.float16, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        gs.gs_unscale_check([g[::2]], [torch.zeros(50, device=dev)], torch.ones(1, device=dev),
                            torch.zeros(1, dtype=torch.int32, device=dev))


def test_given_stream_is_used(dev):
    """A torch stream passed explicitly carries the launch (checked by
    ordering: the result is complete once that stream alone is synchronised)."""
    s = torch.cuda.Stream(device=dev)
    x = torch.ones(128, 256, dtype=torch.bfloat16, device=dev)
    s.wait_stream(torch.cuda.current_stream())
    codes, scales = gs.fp8_quantize(x, E4M3, B1, stream=s)
    out = gs.fp8_dequantize(codes, E4M3, B1, scales, stream=s)
    s.synchronize()
    assert bool((out == 1.0).all())
