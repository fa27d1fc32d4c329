"""Pins of the oracle's BF16 dequantize (the FP32 dequantized value rounded
once more to BF16, nearest with ties to even; canonical NaN 0x7FC0), against
torch on the CPU: the codes decoded by torch's float8 types, multiplied by
the block scale in torch float32, and cast by torch to bfloat16 (its
round-to-nearest-even conversion).  ("Mixed precision and FP8 training", FP8
training section: quant() casts back to float and multiplies by the scale;
the BF16 result is the same value in the BF16 compute type.)"""
import numpy as np
import pytest
import torch

import oracle

FP8 = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}


def _torch_ref(codes, fmt, s_per_elem):
    v = torch.from_numpy(codes).view(FP8[fmt]).float()
    y = v * torch.from_numpy(s_per_elem.astype(np.float32))
    b = y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    b[torch.isnan(y).numpy()] = 0x7FC0
    return b


SPECIAL_SCALES = np.float32([1.0, 0.5, 3.0, 1e-3, 2.0 ** -126, 1e-40, 1e-45, 0.0, -2.0,
                             3.0e38, 1.7e38, np.inf, -np.inf, np.nan, 65536.0, 7.0e-31])


@pytest.mark.parametrize("fmt", [0, 1])
def test_all_codes_times_special_and_random_scales_1x128(fmt):
    rng = np.random.default_rng(900 + fmt)
    rand = rng.integers(0, 1 << 32, size=240, dtype=np.uint64).astype(np.uint32).view(np.float32)
    scales = np.concatenate([SPECIAL_SCALES, rand]).astype(np.float32)
    rows = scales.size
    codes = np.tile(np.arange(256, dtype=np.uint16).astype(np.uint8), (rows, 1))  # 2 blocks per row
    sc = np.repeat(scales, 2)                                                        # [rows][2]
    got = oracle.dequantize_bf16(codes, fmt, oracle.BLOCK_1x128, sc)
    want = _torch_ref(codes, fmt, np.repeat(scales[:, None], 256, axis=1))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("gran", [oracle.PER_TENSOR, oracle.BLOCK_128x128, oracle.BLOCK_1x32])
def test_other_granularities(gran):
    rng = np.random.default_rng(910 + gran)
    rows, cols = (37, 53) if gran == oracle.PER_TENSOR else (256, 384) if gran == oracle.BLOCK_128x128 \
        else (5, 96)
    codes = rng.integers(0, 256, size=(rows, cols), dtype=np.uint16).astype(np.uint8)
    ns = oracle.n_scales(rows, cols, gran)
    sc = np.ldexp(rng.uniform(0.5, 2.0, ns), rng.integers(-100, 100, ns)).astype(np.float32)
    if gran == oracle.PER_TENSOR:
        s = np.full((rows, cols), sc[0], np.float32)
    elif gran == oracle.BLOCK_128x128:
        s = np.kron(sc.reshape(rows // 128, cols // 128), np.ones((128, 128), np.float32))
    else:
        s = np.repeat(sc.reshape(rows, cols // 32), 32, axis=1)
    for fmt in (0, 1):
        got = oracle.dequantize_bf16(codes, fmt, gran, sc)
        assert np.array_equal(got, _torch_ref(codes, fmt, s))


def test_rounding_edges():
    """Ties and overflow at the BF16 grid, built from E4M3 code 0x38 (1.0):
    s = 1 + k * 2^-8 puts 1.0 * s exactly on a tie between two BF16 values
    (odd k: the even neighbour wins), and s just below FP32's maximum rounds
    to +Inf, the largest BF16 being below it."""
    ks = np.arange(-64, 65)
    s = (1.0 + ks * 2.0 ** -8).astype(np.float32)
    s = np.concatenate([s, np.float32([3.4028235e38, 3.3961776e38, 3.3895314e38])])
    codes = np.full((s.size, 32), 0x38, np.uint8)
    got = oracle.dequantize_bf16(codes, 0, oracle.BLOCK_1x32, s)
    want = _torch_ref(codes, 0, np.repeat(s[:, None], 32, axis=1))
    assert np.array_equal(got, want)
    assert got[-3, 0] == 0x7F80          # FP32 max rounds up to +Inf in BF16
