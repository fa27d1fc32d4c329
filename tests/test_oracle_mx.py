"""Pins of the oracle's MX-style 1x32 quantizer with power-of-two (E8M0)
scales.  "Mixed precision and FP8 training" (hardware notes) says only that
MX formats keep one scale per 32 elements; the reading is the page's own
per_block listing on 1x32 blocks with its scale rounded up to a power of
two and stored as the E8M0 byte (2^(byte-127)).  Pinned by the listing run
by torch CPU with that scale (torch.frexp rounds it), by the byte being the
FP32 exponent field of that power of two, and by properties."""
import numpy as np
import pytest
import torch

import oracle

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def _listing_mx(x: torch.Tensor, fmt: int):
    """per_block(x, 1, 32) of the page's fp8_scaling.py, with the scale
    replaced by the smallest power of two not below it."""
    MAX = torch.finfo(TORCH_FP8[fmt]).max
    R, C = x.shape
    b = x.reshape(R, C // 32, 32)
    s = b.abs().amax(dim=2, keepdim=True).clamp(min=1e-12) / MAX
    m, e = torch.frexp(s)
    s2 = torch.where(m == 0.5, s, torch.ldexp(torch.ones_like(s), e))
    codes = (b / s2).clamp(-MAX, MAX).to(TORCH_FP8[fmt]).reshape(R, C)
    return codes.view(torch.uint8).numpy(), s2.reshape(R, C // 32).numpy(), s.reshape(R, C // 32).numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matches_listing_with_power_of_two_scale(fmt, dtype):
    g = torch.Generator().manual_seed(7 + fmt)
    x = torch.randn(96, 256, generator=g)
    x[:, :2] *= 500.0
    x[3, 40:72] *= 1e-20                      # a whole quiet block
    x[5, 0:32] = 0.0                          # an all-zero block: the floor
    x[6, 64:96] = torch.ldexp(torch.ones(32), torch.arange(-16, 16))   # amax exactly 2^15
    x[8, 9] = -0.0
    if dtype == "bf16":
        bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        xf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
        codes, sc, nf = oracle.quantize_mx(bits, fmt)
    else:
        xf = x
        codes, sc, nf = oracle.quantize_mx(x.numpy(), fmt)
    ref_codes, s2, s = _listing_mx(xf, fmt)
    assert np.array_equal(codes, ref_codes)
    # the byte is the FP32 exponent field of the power of two (E8M0 bias 127 = FP32 bias)
    assert np.array_equal(sc, (s2.view(np.uint32) >> 23).astype(np.uint8))
    assert np.all((s2.view(np.uint32) & 0x7FFFFF) == 0)
    assert np.all((s <= s2) & (s2 < 2 * s))
    assert nf == 0
    deq = oracle.dequantize_mx(codes, fmt, sc)
    ref = (torch.from_numpy(ref_codes).view(TORCH_FP8[fmt]).float().reshape(96, 8, 32) *
           torch.from_numpy(s2).reshape(96, 8, 1)).reshape(96, 256).numpy()
    assert np.array_equal(deq.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_no_saturation_and_full_use_of_range(fmt):
    """Like the page's scale, the power of two never clips a finite value,
    and it wastes less than one binade: the block max lands in (MAX/2, MAX]."""
    MAX = oracle.FMT_MAX[fmt]
    x = (np.random.default_rng(2).standard_normal((64, 512)) *
         np.exp(np.random.default_rng(3).uniform(-20, 20, (64, 1)))).astype(np.float32)
    codes, sc, _ = oracle.quantize_mx(x, fmt)
    deq = oracle.dequantize_mx(codes, fmt, sc)
    s = np.ldexp(1.0, sc.astype(np.int32) - 127)
    xb = np.abs(x.reshape(64, 16, 32)).max(axis=2)
    q = xb / s
    assert np.all(q <= MAX) and np.all(q > MAX / 2)
    blk = np.abs(deq.reshape(64, 16, 32)).max(axis=2) / s
    assert np.all(blk <= MAX)


def test_power_of_two_invariance():
    x = np.random.default_rng(4).standard_normal((32, 128)).astype(np.float32)
    c0, s0, _ = oracle.quantize_mx(x, E4M3)
    for k in (-30, -1, 1, 17):
        ck, sk, _ = oracle.quantize_mx((x * np.float32(2.0 ** k)).astype(np.float32), E4M3)
        assert np.array_equal(ck, c0) and np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_nan_scale_byte_and_extreme_bytes():
    codes = np.tile(np.arange(256, dtype=np.uint8)[None, :], (3, 1))     # 3 x 256
    sc = np.zeros((3, 8), np.uint8)
    sc[0, :] = 0xFF
    sc[1, :] = 0
    sc[2, :] = 254
    out = oracle.dequantize_mx(codes, E5M2, sc)
    assert np.all(out[0].view(np.uint32) == oracle.CANONICAL_NAN_BITS)
    v = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e5m2).float()
    for row, b in ((1, 0), (2, 254)):
        ref = (v * torch.ldexp(torch.tensor(1.0), torch.tensor(b - 127))).numpy()
        ref = np.where(np.isnan(ref), np.float32(np.nan), ref).astype(np.float32)
        got = out[row]
        fin = ~np.isnan(ref)
        assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
        assert np.all(got[~fin].view(np.uint32) == oracle.CANONICAL_NAN_BITS)


def test_cols_must_be_multiple_of_32():
    with pytest.raises(ValueError):
        oracle.quantize_mx(np.zeros((2, 48), np.float32), E4M3)
