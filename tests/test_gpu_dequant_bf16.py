"""GPU parity of the BF16 dequantize through the C ABI, bit for bit against
the oracle: all 256 codes of both formats times special and random scales at
every FP32-scale granularity, per-tensor shapes with a ragged tail (element
counts not a multiple of 4), quantize -> BF16 dequantize round trips, and
sampled rows and tiles at the DeepSeek-V3 activation and weight shapes."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu

PT, B1, B128, B32 = gs.FP8_PER_TENSOR, gs.FP8_BLOCK_1x128, gs.FP8_BLOCK_128x128, gs.FP8_BLOCK_1x32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(codes_h, fmt, gran, scales_h, dev):
    c = torch.from_numpy(codes_h).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(scales_h, np.float32)).to(dev)
    out = gs.fp8_dequantize_bf16(c, fmt, gran, s)
    torch.cuda.synchronize()
    return _bits(out)


SPECIAL = np.float32([1.0, 0.5, 3.0, 1e-3, 2.0 ** -126, 1e-40, 1e-45, 0.0, -2.0, 3.0e38,
                      1.7e38, np.inf, -np.inf, np.nan, 65536.0, 7.0e-31])


@pytest.mark.parametrize("fmt", [0, 1])
def test_all_codes_times_scales(fmt, dev):
    rng = np.random.default_rng(950 + fmt)
    rand = rng.integers(0, 1 << 32, size=496, dtype=np.uint64).astype(np.uint32).view(np.float32)
    scales = np.concatenate([SPECIAL, rand]).astype(np.float32)          # 512 scales
    # 1x128: 256 rows of 256 codes (two blocks per row)
    codes = np.tile(np.arange(256, dtype=np.uint16).astype(np.uint8), (256, 1))
    sc = scales.reshape(256, 2)
    assert np.array_equal(_run(codes, fmt, B1, sc, dev), oracle.dequantize_bf16(codes, fmt, B1, sc))
    # 1x32: 64 rows x 256 codes = 8 blocks per row
    codes = np.tile(np.arange(256, dtype=np.uint16).astype(np.uint8), (64, 1))
    sc = scales.reshape(64, 8)
    assert np.array_equal(_run(codes, fmt, B32, sc, dev), oracle.dequantize_bf16(codes, fmt, B32, sc))
    # 128x128: a 512 x 1024 matrix of codes (32 tiles), one scale per tile
    codes = rng.integers(0, 256, size=(512, 1024), dtype=np.uint16).astype(np.uint8)
    sc = scales[:32].reshape(4, 8)
    assert np.array_equal(_run(codes, fmt, B128, sc, dev),
                          oracle.dequantize_bf16(codes, fmt, B128, sc))
    # per-tensor: every scale on the 256 codes
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8).reshape(16, 16)
    for s in scales[:64]:
        sc = np.float32([s])
        assert np.array_equal(_run(codes, fmt, PT, sc, dev),
                              oracle.dequantize_bf16(codes, fmt, PT, sc)), s


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (7, 129), (1000, 999), (1024, 1027)])
def test_per_tensor_ragged_tails(shape, dev):
    rng = np.random.default_rng(960 + shape[1])
    codes = rng.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    for fmt in (0, 1):
        sc = np.float32([rng.uniform(0.001, 100.0)])
        assert np.array_equal(_run(codes, fmt, PT, sc, dev), oracle.dequantize_bf16(codes, fmt, PT, sc))


def test_quantize_then_bf16_dequantize(dev):
    """Round trips of seeded BF16 data with planted specials through the
    quantizer (scales from the block amax) and the BF16 dequantizer."""
    rng = np.random.default_rng(970)
    for gran, (rows, cols) in ((B1, (384, 1024)), (B128, (384, 640)), (B32, (300, 608)),
                               (PT, (257, 333))):
        x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
        x.reshape(-1)[rng.choice(x.size, 50, replace=False)] = \
            rng.choice(np.float32([np.nan, np.inf, -np.inf, 0.0, 1e4]), 50)
        b = x.view(np.uint32)
        xh = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
        xh[np.isnan(x)] = 0x7FC0
        xd = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
        for fmt in (0, 1):
            codes, sc = gs.fp8_quantize(xd, fmt, gran)
            out = gs.fp8_dequantize_bf16(codes, fmt, gran, sc)
            torch.cuda.synchronize()
            rc, rs, _ = oracle.quantize(xh, fmt, gran)
            assert np.array_equal(_bits(out), oracle.dequantize_bf16(rc, fmt, gran, rs)), (gran, fmt)


def test_full_size_sampled(dev):
    """The DeepSeek-V3 activation (16384x7168, 1x128) and weight (7168x18432,
    128x128) shapes: GPU codes and scales from the quantizer, the BF16
    dequantize of the whole matrix on the GPU, and the oracle's BF16
    dequantize of 64 sampled rows (activation) and 2 sampled 128-row slabs
    of tiles (weight) from the same codes and scales."""
    act, wgt = synth.deepseek_v3_blocks()
    rng = np.random.default_rng(980)
    for sp, gran in ((act, B1), (wgt, B128)):
        x = sp.full(dev)
        codes, sc = gs.fp8_quantize(x, sp.fmt, gran)
        out = gs.fp8_dequantize_bf16(codes, sp.fmt, gran, sc)
        torch.cuda.synchronize()
        if gran == B1:
            rows = np.sort(rng.choice(sp.rows, 64, replace=False))
            c = codes[rows].cpu().numpy()
            s = sc[rows].cpu().numpy()
            got = _bits(out[rows])
            assert np.array_equal(got, oracle.dequantize_bf16(c, sp.fmt, B1, s))
        else:
            for ti in rng.choice(sp.rows // 128, 2, replace=False):
                r0 = int(ti) * 128
                c = codes[r0:r0 + 128].cpu().numpy()
                s = sc[int(ti):int(ti) + 1].cpu().numpy()
                got = _bits(out[r0:r0 + 128])
                assert np.array_equal(got, oracle.dequantize_bf16(c, sp.fmt, B128, s))
        del x, codes, sc, out
