"""Pins of the oracle's number-format codecs (CPU only).

Each test ties the oracle to something other than itself: constants the pages
print, the closed-form definition of the OCP FP8 formats, and library
routines (numpy's IEEE half widening, torch CPU's float8 casts) over the
whole input space.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden

E4M3, E5M2 = oracle.E4M3, oracle.E5M2
TORCH_FP8 = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def _floats(s):
    return [float(v) for v in s.split(",")]


# ------------------------------------------------------------------ constants
def test_fp8_constants_match_pages():
    g = load_golden("format_constants.txt")
    d4 = oracle.fp8_decode_table(E4M3)
    d5 = oracle.fp8_decode_table(E5M2)
    # max normal: 448 = code 0x7E, 57344 = code 0x7B; nothing finite above
    assert d4[0x7E] == float(g["e4m3_max"]) == np.nanmax(d4[np.isfinite(d4)])
    assert d5[0x7B] == float(g["e5m2_max"]) == np.nanmax(d5[np.isfinite(d5)])
    # bias: the exponent field equal to the bias encodes 2^0
    assert d4[int(g["e4m3_bias"]) << 3] == 1.0
    assert d5[int(g["e5m2_bias"]) << 2] == 1.0
    # smallest normal / subnormal of E4M3 (fp8_scaling.py output; exercise answer)
    assert d4[0x08] == float(g["e4m3_min_normal"])
    assert d4[0x01] == float(g["e4m3_min_subnormal"]) == 2.0 ** -9
    assert d5[0x04] == 2.0 ** -14 and d5[0x01] == 2.0 ** -16
    # E4M3: no infinities, exactly one NaN mantissa pattern per sign
    assert not np.isinf(d4).any()
    assert sorted(np.flatnonzero(np.isnan(d4)).tolist()) == [0x7F, 0xFF]
    # E5M2: IEEE-style specials
    assert d5[0x7C] == math.inf and d5[0xFC] == -math.inf
    assert sorted(np.flatnonzero(np.isnan(d5)).tolist()) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]


def test_e4m3_binade_count():
    """18 binades for OCP E4M3; an IEEE-style E4M3 that reserved exponent 15
    for infinities would keep only 17."""
    g = load_golden("format_constants.txt")
    d4 = oracle.fp8_decode_table(E4M3)
    pos = d4[1:0x7F]                        # positive finite nonzero codes
    binades = {math.floor(math.log2(v)) for v in pos}
    assert len(binades) == int(g["e4m3_binades"])
    ieee_like = {math.floor(math.log2(d4[c])) for c in range(1, 0x78)}  # exponent < 15
    assert len(ieee_like) == int(g["e4m3_ieee_style_binades"])


def test_fp16_constants_match_pages():
    g = load_golden("format_constants.txt")
    w = oracle.f16_to_f32(np.array([0x7BFF, 0x0400, 0x0001, 0x3C00, 0x3C01], np.uint16))
    assert w[0] == float(g["fp16_max"]) == 65504.0
    assert w[1] == 2.0 ** -14 and float("%.3g" % w[1]) == float(g["fp16_min_normal"])
    assert w[2] == 2.0 ** -24 and float("%.3g" % w[2]) == float(g["fp16_min_subnormal"])
    assert w[3] == 1.0


def test_finfo_rows_of_precision_py():
    """The precision.py finfo lines: max, smallest normal and eps, printed with
    3 significant digits, derived from the oracle's own widening codecs."""
    g = load_golden("precision_py.txt")
    h = oracle.f16_to_f32(np.array([0x7BFF, 0x0400, 0x3C01], np.uint16)).astype(np.float64)
    fp16 = [h[0], h[1], h[2] - 1.0]
    bf = oracle.bf16_to_f32(np.array([0x7F7F, 0x0080, 0x3F81], np.uint16)).astype(np.float64)
    bf16 = [bf[0], bf[1], bf[2] - 1.0]
    for row, vals in (("fp16_finfo", fp16), ("bf16_finfo", bf16)):
        assert ["%.3g" % v for v in vals] == [s.strip() for s in g[row].split(",")]


# ------------------------------------------------------------------ FP16 widening
def test_f16_widening_all_patterns_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


# ------------------------------------------------------------------ FP8 decode
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_decode_all_codes_vs_torch(fmt):
    ours = oracle.fp8_decode_table(fmt)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(TORCH_FP8[fmt]).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN lanes: same class and sign (payloads differ between libraries)
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


# ------------------------------------------------------------------ FP8 encode
def _torch_encode(y: np.ndarray, fmt: int) -> np.ndarray:
    m = oracle.FMT_MAX[fmt]
    t = torch.from_numpy(y)
    return t.clamp(-m, m).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()


def _grid_neighbourhood(fmt: int) -> np.ndarray:
    """Every FP8 value and every midpoint between neighbours, each with its
    FP32 neighbours at +-1 and +-2 ulp, both signs, plus values around MAX
    and the subnormal edge: the inputs where a wrong rounding rule shows."""
    vals = oracle.fp8_decode_table(fmt)
    fin = np.sort(np.unique(vals[np.isfinite(vals) & (vals >= 0)]))
    mids = (fin[1:] + fin[:-1]) / 2
    pts = np.concatenate([fin, mids, [oracle.FMT_MAX[fmt] * k for k in (1.0, 1.0625, 1.125, 2.0)]])
    base = pts.astype(np.float32).view(np.int32)
    around = np.concatenate([base + d for d in (-2, -1, 0, 1, 2)])
    around = around[around >= 0].view(np.float32)
    return np.concatenate([around, -around, np.float32([np.inf, -np.inf, 0.0, -0.0])])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_encode_grid_and_random_vs_torch(fmt):
    rng = np.random.default_rng(1234 + fmt)
    rand_bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    y = np.concatenate([_grid_neighbourhood(fmt), rand_bits.view(np.float32)])
    assert np.array_equal(oracle.fp8_encode(y, fmt), _torch_encode(y, fmt))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_encode_every_fp32_pattern_vs_torch(fmt):
    """All 2^32 FP32 bit patterns, NaN codes included (torch also writes
    sign|0x7F for a NaN input)."""
    chunk = 1 << 26
    for lo in range(0, 1 << 32, chunk):
        y = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        ours = oracle.fp8_encode(y, fmt)
        ref = _torch_encode(y, fmt)
        if not np.array_equal(ours, ref):
            bad = np.flatnonzero(ours != ref)[:8]
            raise AssertionError("mismatch at bit patterns %s" % [hex(lo + int(i)) for i in bad])


def test_fp8_roundtrip_all_codes():
    """encode(decode(c)) == c for every E4M3 code; for E5M2 the identity
    holds except that Inf saturates to MAX and NaN codes canonicalise to
    sign|0x7F."""
    for fmt in (E4M3, E5M2):
        dec = oracle.fp8_decode_table(fmt).astype(np.float32)
        enc = oracle.fp8_encode(dec, fmt)
        codes = np.arange(256)
        expect = codes.copy()
        if fmt == E5M2:
            expect[0x7C], expect[0xFC] = 0x7B, 0xFB
            expect[[0x7D, 0x7E]] = 0x7F
            expect[[0xFD, 0xFE]] = 0xFF
        assert np.array_equal(enc, expect.astype(np.uint8)), fmt


def test_fp8_encode_ties_to_even_and_saturation():
    # E4M3: 2^-10 is halfway between 0 and 2^-9 -> 0 (even); 3*2^-10 -> 2*2^-9
    # E5M2: 480 is halfway between 448 and 512 -> 512 (mantissa 00 is even)
    e4 = oracle.fp8_encode(np.float32([2 ** -10, 3 * 2 ** -10, -(2 ** -10), 1e30, -np.inf]), E4M3)
    assert e4.tolist() == [0x00, 0x02, 0x80, 0x7E, 0xFE]
    e5 = oracle.fp8_encode(np.float32([480.0, 57344 * 1.125, 2 ** -17, 3 * 2 ** -17]), E5M2)
    assert e5.tolist() == [0x60, 0x7B, 0x00, 0x02]
