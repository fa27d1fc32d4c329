"""The Python binding's own argument checks, on the CPU: host tensors are
refused before anything reaches the C ABI (whose bare pointers would send a
host address to a kernel), for every entry point."""
import pytest
import torch

import loss_scaling_fp8_amd as gs

BF16, F32 = torch.bfloat16, torch.float32


def _host_calls():
    x = torch.zeros(4, 128, dtype=BF16)
    codes = torch.zeros(4, 128, dtype=torch.uint8)
    sc = torch.ones(4, 1, dtype=F32)
    S = torch.ones(1, dtype=F32)
    i32 = torch.zeros(1, dtype=torch.int32)
    g, o = torch.zeros(8, dtype=torch.float16), torch.zeros(8, dtype=F32)
    return {
        "gs_unscale_check": lambda: gs.gs_unscale_check([g], [o], S, i32),
        "gs_unscale_check_sumsq": lambda: gs.gs_unscale_check_sumsq(
            [g], [o], S, i32, torch.zeros(2, dtype=torch.int64), torch.zeros(1, dtype=torch.float64)),
        "gs_update_scale": lambda: gs.gs_update_scale(S, i32, i32),
        "gs_update_scale_hysteresis": lambda: gs.gs_update_scale_hysteresis(S, i32, i32, i32),
        "fp8_quantize": lambda: gs.fp8_quantize(x, gs.FP8_E4M3, gs.FP8_BLOCK_1x128),
        "fp8_quantize_no_workspace": lambda: gs.fp8_quantize_no_workspace(
            x, gs.FP8_E4M3, gs.FP8_PER_TENSOR, codes, S),
        "fp8_quantize_delayed": lambda: gs.fp8_quantize_delayed(
            x, gs.FP8_E4M3, S, torch.zeros(4, dtype=F32), i32),
        "fp8_dequantize": lambda: gs.fp8_dequantize(codes, gs.FP8_E4M3, gs.FP8_BLOCK_1x128, sc),
        "fp8_dequantize_bf16": lambda: gs.fp8_dequantize_bf16(codes, gs.FP8_E4M3, gs.FP8_BLOCK_1x128, sc),
        "fp8_quantize_mx": lambda: gs.fp8_quantize_mx(x, gs.FP8_E4M3),
        "fp8_dequantize_mx": lambda: gs.fp8_dequantize_mx(
            codes, gs.FP8_E4M3, torch.zeros(4, 4, dtype=torch.uint8)),
    }


@pytest.mark.parametrize("entry", sorted(_host_calls()))
def test_host_tensors_are_refused(entry):
    with pytest.raises(ValueError, match="must be on a GPU"):
        _host_calls()[entry]()


def test_every_tensor_entry_point_is_covered():
    names = set(gs.EXPORTS) - {"gs_unscale_list_descriptors", "gs_status_string",
                               "gs_unscale_check_sumsq_workspace_size",
                               "fp8_quantize_workspace_size"}
    assert names == set(_host_calls())


def test_non_tensor_arguments_are_refused():
    with pytest.raises(TypeError):
        gs.fp8_quantize([[1.0]], gs.FP8_E4M3, gs.FP8_PER_TENSOR)
    with pytest.raises(ValueError, match="scale is required"):
        gs.gs_unscale_check([], [], None, None)
