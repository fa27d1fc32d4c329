"""Property tests of the oracle with hypothesis (CPU; derandomized, no example
database), each against something other than the oracle's own formula:

* the unscale against numpy's IEEE float32 arithmetic (fl32(f) * fl32(1/S),
  canonical NaN, the flag iff any output is not finite);
* the exact sum of squares against Python's arbitrary-precision integers;
* the quantizer's invariants ("Mixed precision and FP8 training", FP8
  training section, quant / per_tensor / per_block): codes unchanged and
  scales exactly times 2^k when the input is scaled by 2^k, codes monotone
  within a block, and the round-trip error within half an FP8 spacing of
  the quotient times s (plus the FP32 roundings)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))
CANON = 0x7FC00000
GRANS = [oracle.PER_TENSOR, oracle.BLOCK_1x128, oracle.BLOCK_128x128, oracle.BLOCK_1x32]


def _bf16(x):
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


scales = st.one_of(st.integers(-30, 40).map(lambda k: float(np.ldexp(np.float32(1), k))),
                   st.floats(1e-3, 1e6).map(lambda v: float(np.float32(v))))
fp16_lists = st.lists(st.lists(st.integers(0, 0xFFFF), max_size=300), max_size=5)


@SETTINGS
@given(fp16_lists, scales)
def test_unscale_matches_numpy_float32(grads, S):
    hs = [np.array(g, dtype=np.uint16) for g in grads]
    outs, flag = oracle.unscale_check(hs, S)
    inv = np.float32(1) / np.float32(S)
    any_bad = False
    for h, o in zip(hs, outs):
        with np.errstate(invalid="ignore", over="ignore"):
            y = h.view(np.float16).astype(np.float32) * inv
        bits = y.view(np.uint32).copy()
        bits[np.isnan(y)] = CANON
        assert np.array_equal(o.view(np.uint32), bits)
        any_bad |= bool((~np.isfinite(y)).any())
    assert flag == int(any_bad)


@SETTINGS
@given(fp16_lists, scales, st.integers(0, (1 << 100)))
def test_sum_of_squares_is_the_exact_integer(grads, S, start):
    hs = [np.array(g, dtype=np.uint16) for g in grads]
    start_pair = (start & ((1 << 64) - 1), start >> 64)
    _, _, acc, _ = oracle.unscale_check_sumsq(hs, S, sumsq=start_pair)
    X = start
    for h in hs:
        for v in h.view(np.float16).astype(np.float64):
            if np.isfinite(v):
                q = int(abs(v) * 2.0 ** 24)        # exact: every finite FP16 is a multiple of 2^-24
                X += q * q
    X %= 1 << 128
    assert (acc[0], acc[1]) == (X & ((1 << 64) - 1), X >> 64)


def _shape(gran, r, c):
    if gran == oracle.BLOCK_1x128:
        return r % 4 + 1, 128 * (c % 3 + 1)
    if gran == oracle.BLOCK_128x128:
        return 128, 128 * (c % 2 + 1)
    if gran == oracle.BLOCK_1x32:
        return r % 4 + 1, 32 * (c % 4 + 1)
    return r % 20 + 1, c % 40 + 1


@st.composite
def block_inputs(draw):
    gran = draw(st.sampled_from(GRANS))
    rows, cols = _shape(gran, draw(st.integers(0, 1000)), draw(st.integers(0, 1000)))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    mag = np.ldexp(rng.uniform(1.0, 2.0, (rows, cols)), rng.integers(-20, 21, (rows, cols)))
    x = (mag * rng.choice([-1.0, 1.0], (rows, cols))).astype(np.float32)
    dtype = draw(st.sampled_from(["bf16", "f32"]))
    return gran, (_bf16(x) if dtype == "bf16" else x), draw(st.integers(0, 1))


def _as_f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x


@SETTINGS
@given(block_inputs(), st.integers(-20, 20))
def test_scaling_the_input_by_2k_scales_the_scales_exactly(inp, k):
    gran, x, fmt = inp
    c0, s0, _ = oracle.quantize(x, fmt, gran)
    if x.dtype == np.uint16:
        xb = x.astype(np.int32) + (k << 7)                   # BF16 exponent field + k
        xk = (xb & 0xFFFF).astype(np.uint16)
    else:
        xk = np.ldexp(x, k).astype(np.float32)
    c1, s1, _ = oracle.quantize(xk, fmt, gran)
    assert np.array_equal(c0, c1)
    assert np.array_equal(np.ldexp(s0.astype(np.float64), k), s1.astype(np.float64))


def _spacing(y, fmt):
    """FP8 spacing at |y| (E4M3: 3 fraction bits, min exponent -6; E5M2: 2, -14)."""
    m, emin = (3, -6) if fmt == 0 else (2, -14)
    e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 1e-300))), emin)
    return np.ldexp(1.0, (e - m).astype(np.int64))


@SETTINGS
@given(block_inputs())
def test_codes_monotone_and_error_within_half_spacing(inp):
    gran, x, fmt = inp
    codes, sc, _ = oracle.quantize(x, fmt, gran)
    table = oracle.fp8_decode_table(fmt)
    xf = _as_f32(x).astype(np.float64)
    rows, cols = xf.shape
    # the scale of each element's block
    if gran == oracle.PER_TENSOR:
        s = np.full((rows, cols), sc[0], np.float64)
    elif gran == oracle.BLOCK_1x128:
        s = np.repeat(sc.reshape(rows, cols // 128), 128, axis=1).astype(np.float64)
    elif gran == oracle.BLOCK_1x32:
        s = np.repeat(sc.reshape(rows, cols // 32), 32, axis=1).astype(np.float64)
    else:
        s = np.kron(sc.reshape(rows // 128, cols // 128), np.ones((128, 128))).astype(np.float64)
    v = table[codes]
    # error: within half a spacing of the quotient, plus the two FP32 roundings
    y = xf / s
    err = np.abs(v * s - xf)
    bound = 0.5 * _spacing(y, fmt) * s + 2.0 ** -22 * np.abs(xf)
    assert (err <= bound).all()
    # monotone: within each block, a larger x never gets a smaller value
    blocks = [(slice(None), slice(None))] if gran == oracle.PER_TENSOR else None
    if blocks is None:
        w = 128 if gran in (oracle.BLOCK_1x128, oracle.BLOCK_128x128) else 32
        h = 128 if gran == oracle.BLOCK_128x128 else 1
        blocks = [(slice(i, i + h), slice(j, j + w)) for i in range(0, rows, h)
                  for j in range(0, cols, w)]
    for b in blocks:
        xs, vs = xf[b].reshape(-1), v[b].reshape(-1)
        order = np.argsort(xs, kind="stable")
        assert (np.diff(vs[order]) >= 0).all()
