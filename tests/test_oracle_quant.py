"""Pins of the oracle's FP8 quantizer and dequantizer (CPU only).

The fp8_scaling.py listing of 'Mixed precision and FP8 training' (section
'FP8 training') is itself a torch CPU program: on finite FP32 data it is the
library routine the oracle must reproduce bit for bit (codes, scales and the
dequantized values).  The printed error table and the outlier exercise pin
the whole quantize + dequantize round trip; the remaining tests check
properties that follow from the definition at any size.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
PT, B1, B128, B32 = oracle.PER_TENSOR, oracle.BLOCK_1x128, oracle.BLOCK_128x128, oracle.BLOCK_1x32
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
BLOCK = {PT: None, B1: (1, 128), B128: (128, 128), B32: (1, 32)}


def _floats(s):
    return [float(v) for v in s.split(",")]


# ---- the page's per-block rule, block by block with torch CPU primitives
def _blocks(shape, gran):
    """(row slice, column slice) of every block, in the row-major order of
    the scale layout."""
    R, C = shape
    br, bc = BLOCK[gran] or (R, C)
    return [(slice(r0, r0 + br), slice(c0, c0 + bc))
            for r0 in range(0, R, br) for c0 in range(0, C, bc)]


def _listing_codes_and_scales(x: torch.Tensor, fmt: int, gran: int):
    """For each block: its largest |x| (the 1e-12 floor applies to blocks;
    the page's per-tensor function has none, and these inputs never need
    it), the FP32 scale amax / MAX, then each element divided by the scale,
    clamped to [-MAX, MAX] and cast by torch to the float8 type (round to
    nearest even).  Returns the codes as bytes and the scales in block
    order."""
    fp8 = TORCH_FP8[fmt]
    MAX = float(torch.finfo(fp8).max)
    codes = torch.empty(x.shape, dtype=torch.uint8)
    scales = []
    for rs, cs in _blocks(x.shape, gran):
        block = x[rs, cs]
        amax = block.abs().max()
        if gran != PT:
            amax = torch.clamp(amax, min=1e-12)
        s = amax / MAX
        codes[rs, cs] = torch.clamp(block / s, -MAX, MAX).to(fp8).view(torch.uint8)
        scales.append(s)
    return codes.numpy(), torch.stack(scales).numpy()


def _listing_dequant(codes: np.ndarray, s: np.ndarray, fmt: int, gran: int):
    """Each block's codes decoded by torch (float8 to float32) times its
    scale."""
    q = torch.from_numpy(codes).view(TORCH_FP8[fmt]).float()
    out = torch.empty(q.shape, dtype=torch.float32)
    for k, (rs, cs) in enumerate(_blocks(q.shape, gran)):
        out[rs, cs] = q[rs, cs] * float(s[k])
    return out.numpy()


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("gran", [PT, B1, B128, B32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_matches_page_listing(fmt, gran, dtype):
    g = torch.Generator().manual_seed(100 + 10 * fmt + gran)
    x = torch.randn(256, 512, generator=g)
    x[:, :3] *= 300.0
    x[7, 200] = 1e-30                      # deep underflow in every block size
    x[9, 9] = -0.0
    x[130:135, 256:384] *= 1e-6            # a quiet block next to loud ones
    if dtype == "bf16":
        bits = _bf16_bits(x)
        xf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()  # exact widening
        ours = oracle.quantize(bits, fmt, gran)
    else:
        xf = x
        ours = oracle.quantize(x.numpy(), fmt, gran)
    ref_codes, ref_s = _listing_codes_and_scales(xf, fmt, gran)
    assert np.array_equal(ours[1].view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(ours[0], ref_codes)
    assert ours[2] == 0
    deq = oracle.dequantize(ours[0], fmt, gran, ours[1])
    assert np.array_equal(deq.view(np.uint32), _listing_dequant(ref_codes, ref_s, fmt, gran).view(np.uint32))


def test_page_error_table():
    """The printed table: relative error on ordinary channels, per-tensor vs
    1x128, E4M3, outliers x100 / x1e4 / x3e4 (torch.manual_seed(0))."""
    g = load_golden("fp8_error_table.txt")
    torch.manual_seed(0)
    pt_pct, b_pct = [], []
    for outlier in _floats(g["outliers"]):
        a = torch.randn(256, 1024)
        a[:, :4] *= outlier
        x = a.numpy()
        normal = x[:, 128:].astype(np.float64)
        for gran, acc in ((PT, pt_pct), (B1, b_pct)):
            codes, s, _ = oracle.quantize(x, E4M3, gran)
            q = oracle.dequantize(codes, E4M3, gran, s)[:, 128:].astype(np.float64)
            acc.append(round(100 * np.linalg.norm(q - normal) / np.linalg.norm(normal), 1))
    assert pt_pct == _floats(g["per_tensor_pct"])
    assert b_pct == _floats(g["per_1x128_pct"])


def test_page_outlier_exercise():
    g = load_golden("outlier_exercise.txt")
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, size=(4, 256)).astype(np.float32)
    x[2, 17] = float(g["amax"])
    x[0, 0] = float(g["probe"])
    codes, s, _ = oracle.quantize(x, E4M3, PT)
    assert s[0] == np.float32(5000.0) / np.float32(448.0)
    assert round(float(s[0]), 1) == float(g["scale_approx"])
    assert round(float(g["probe"]) / float(s[0]), 4) == float(g["probe_over_scale"])
    assert float(g["probe"]) / float(s[0]) < float(g["e4m3_min_subnormal"]) / 2
    assert codes[0, 0] == 0x00
    assert oracle.dequantize(codes, E4M3, PT, s)[0, 0] == float(g["probe_code_value"])


# ---------------------------------------------------------------- properties
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("gran", [PT, B1, B128, B32])
def test_scale_invariance_power_of_two(fmt, gran):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((256, 256)) * 3).astype(np.float32)
    c0, s0, _ = oracle.quantize(x, fmt, gran)
    for k in (-20, -3, 5, 40):
        c1, s1, _ = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32), fmt, gran)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** k)).astype(np.float32))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_monotone_and_error_bound(fmt):
    """Within one scale block decode(code) is monotone in x, and for |x/s|
    within range the error is at most half an FP8 spacing (times s) plus the
    two FP32 roundings of x/s and of decode*s."""
    rng = np.random.default_rng(12)
    x = np.sort(rng.standard_normal(128 * 64).astype(np.float32) * 5).reshape(1, -1)
    x = np.ascontiguousarray(x)
    codes, s, _ = oracle.quantize(x, fmt, PT)
    dec = oracle.fp8_decode_table(fmt)[codes[0]]
    assert (np.diff(dec) >= 0).all()
    q = oracle.dequantize(codes, fmt, PT, s)[0].astype(np.float64)
    sv = float(s[0])
    y = x[0].astype(np.float64) / sv
    mbits = 3 if fmt == E4M3 else 2
    emin = -6 if fmt == E4M3 else -14
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 1e-300))), emin)
    half_spacing = 0.5 * 2.0 ** (e - mbits)
    bound = (half_spacing + np.abs(y) * 2.0 ** -24) * sv * (1 + 2.0 ** -23) + np.abs(q) * 2.0 ** -24
    assert (np.abs(q - x[0]) <= bound).all()


def test_ordinary_channel_error_independent_of_outlier():
    """1x128: the error on blocks without the outlier does not change with
    the outlier's size (each block has its own scale)."""
    rng = np.random.default_rng(13)
    base = rng.standard_normal((64, 512)).astype(np.float32)
    errs = []
    for k in (1e2, 1e4, 3e4):
        x = base.copy()
        x[:, :4] *= np.float32(k)
        c, s, _ = oracle.quantize(x, E4M3, B1)
        errs.append(oracle.dequantize(c, E4M3, B1, s)[:, 128:].tobytes())
    assert errs[0] == errs[1] == errs[2]


# ---------------------------------------------------------------- reading-defined rules
# (The pages do not cover these; they are readings the oracle defines, checked
# here for internal consistency only.)
def test_special_values_rules():
    f32 = np.float32
    x = np.zeros((1, 128), np.float32)
    x[0, :8] = [np.nan, -np.nan, np.inf, -np.inf, -0.0, 0.0, 1.0, -2.0]
    codes, s, nf = oracle.quantize(x, E4M3, B1)
    assert nf == 1
    assert s[0] == f32(2.0) / f32(448.0)               # finite-only amax
    assert codes[0, :6].tolist() == [0x7F, 0xFF, 0x7E, 0xFE, 0x80, 0x00]
    # all-zero / all-non-finite blocks use the 1e-12 floor at every granularity
    z = np.zeros((128, 128), np.float32)
    for gran in (PT, B1, B128):
        _, sz, _ = oracle.quantize(z, E5M2, gran)
        assert (sz == f32(1e-12) / f32(57344.0)).all()
    # given-scale mode: s = 0 -> +-MAX for finite nonzero, 0x7F for 0/0
    g = np.float32([[1.0, -1.0, 0.0] + [0.0] * 125])
    cg, _, _ = oracle.quantize(g, E4M3, B1, oracle.GIVEN, np.float32([0.0]))
    assert cg[0, :3].tolist() == [0x7E, 0xFE, 0x7F]
    # negative underflow keeps its sign
    t = np.float32([[-1e-30] + [100.0] * 127])
    ct, _, _ = oracle.quantize(t, E4M3, B1)
    assert ct[0, 0] == 0x80


def test_shape_must_divide_into_blocks():
    x = np.zeros((128, 200), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(x, E4M3, B1)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((100, 128), np.float32), E4M3, B128)
    oracle.quantize(np.zeros((3, 5), np.float32), E4M3, PT)   # any shape per-tensor


def test_dequantize_specials():
    codes = np.array([[0x7F, 0xFF, 0x00, 0x80, 0x7E, 0x01]], np.uint8)
    out = oracle.dequantize(codes, E4M3, PT, np.float32([2.0]))
    assert out.view(np.uint32)[0, :2].tolist() == [oracle.CANONICAL_NAN_BITS] * 2
    assert out[0, 2:].tolist() == [0.0, -0.0, 896.0, 2.0 ** -8]
    assert np.signbit(out[0, 3])
    c5 = np.array([[0x7C, 0xFC, 0x7D]], np.uint8)
    o5 = oracle.dequantize(c5, E5M2, PT, np.float32([0.5]))
    assert o5[0, 0] == np.inf and o5[0, 1] == -np.inf
    assert o5.view(np.uint32)[0, 2] == oracle.CANONICAL_NAN_BITS
    o0 = oracle.dequantize(c5, E5M2, PT, np.float32([0.0]))    # Inf * 0 -> NaN
    assert o0.view(np.uint32)[0, 0] == oracle.CANONICAL_NAN_BITS
