"""GPU parity: FP8 quantize / dequantize through the C ABI, bit for bit
against the oracle (codes, scales, dequantized FP32, the nonfinite flag)."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu

E4M3, E5M2 = gs.FP8_E4M3, gs.FP8_E5M2
PT, B1, B128, B32 = gs.FP8_PER_TENSOR, gs.FP8_BLOCK_1x128, gs.FP8_BLOCK_128x128, gs.FP8_BLOCK_1x32


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _u32(t):
    return t.detach().cpu().contiguous().numpy().reshape(-1).view(np.uint32)


def _special_bf16(rng, rows, cols):
    """BF16 bit patterns: N(0,1)-ish body with planted NaN (both signs,
    payloads), +-Inf, +-0, BF16 subnormals, huge values, values above 448 and
    57344, and exact E4M3/E5M2 midpoints at s = 1."""
    x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    n = rows * cols
    flat = bits.reshape(-1)
    pos = rng.permutation(n)
    k = max(1, n // 50)
    specials = [
        lambda m: 0x7FC0 | rng.integers(0, 0x3F, m).astype(np.uint16),          # +NaN
        lambda m: 0xFF80 | rng.integers(1, 0x7F, m).astype(np.uint16),          # -NaN
        lambda m: np.full(m, 0x7F80, np.uint16), lambda m: np.full(m, 0xFF80, np.uint16),
        lambda m: np.full(m, 0x0000, np.uint16), lambda m: np.full(m, 0x8000, np.uint16),
        lambda m: rng.integers(1, 0x80, m).astype(np.uint16),                   # subnormals
        lambda m: rng.integers(0x7000, 0x7F80, m).astype(np.uint16),            # huge
        lambda m: rng.integers(0x43E0, 0x43F8, m).astype(np.uint16),            # ~448..496
        lambda m: rng.integers(0x4760, 0x4778, m).astype(np.uint16),            # ~57344..63488
        lambda m: (0x3C00 + (rng.integers(0, 120, m) << 4 | 0x8)).astype(np.uint16),  # E4M3 mids
        lambda m: (0x3800 + (rng.integers(0, 240, m) << 5 | 0x10)).astype(np.uint16),  # E5M2 mids
    ]
    for j, f in enumerate(specials):
        idx = pos[j * k:(j + 1) * k]
        flat[idx] = f(idx.size) | (flat[idx] & 0x8000 if j >= 6 else 0)
    return bits


def _run(x_host, fmt, gran, mode, dev, scales_host=None):
    """x_host: float32 array or uint16 BF16 bits [rows, cols]."""
    if x_host.dtype == np.uint16:
        x = torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(x_host).to(dev)
    rows, cols = x_host.shape
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    sc = None
    if scales_host is not None:
        sc = torch.from_numpy(scales_host.astype(np.float32)).to(dev).reshape(
            gs.scale_shape(rows, cols, gran))
    codes, scales = gs.fp8_quantize(x, fmt, gran, mode, scales=sc, nonfinite=nf)
    deq = gs.fp8_dequantize(codes, fmt, gran, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), _u32(scales), _u32(deq), int(nf.item())


def _check(x_host, fmt, gran, mode, dev, scales_host=None):
    c, s, d, nf = _run(x_host, fmt, gran, mode, dev, scales_host)
    rc, rs, rnf = oracle.quantize(x_host, fmt, gran, mode, scales_host)
    rd = oracle.dequantize(rc, fmt, gran, rs)
    if not np.array_equal(c, rc):
        bad = np.argwhere(c != rc)[:5]
        raise AssertionError("codes differ at %s: gpu %s oracle %s" % (
            bad.tolist(), [hex(c[tuple(b)]) for b in bad], [hex(rc[tuple(b)]) for b in bad]))
    assert np.array_equal(s, rs.view(np.uint32)), "scales differ"
    assert np.array_equal(d, rd.reshape(-1).view(np.uint32)), "dequantized values differ"
    assert nf == rnf


SHAPES = {PT: [(1, 1), (3, 5), (7, 129), (1000, 999), (1024, 1024)],
          B1: [(1, 128), (3, 384), (130, 256), (257, 640)],
          B128: [(128, 128), (256, 384), (384, 640)],
          B32: [(1, 32), (3, 96), (130, 256), (257, 608)]}


@pytest.mark.parametrize("gran", [PT, B1, B128, B32])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_special_values_all_shapes(gran, fmt, dtype, dev):
    rng = np.random.default_rng(1000 + 10 * gran + fmt)
    for rows, cols in SHAPES[gran]:
        bits = _special_bf16(rng, rows, cols)
        x = bits if dtype == "bf16" else (bits.astype(np.uint32) << 16).view(np.float32)
        _check(np.ascontiguousarray(x), fmt, gran, gs.FP8_SCALE_FROM_AMAX, dev)


@pytest.mark.parametrize("gran", [PT, B1, B128, B32])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_given_scales_including_degenerate(gran, fmt, dev):
    rng = np.random.default_rng(77 + gran + 3 * fmt)
    rows, cols = (256, 384) if gran != PT else (300, 77)
    bits = _special_bf16(rng, rows, cols)
    ns = oracle.n_scales(rows, cols, gran)
    pool = np.float32([1.0, 0.5, 3.0, 1e-3, 1e-30, 2.0 ** -90, 1e36, 3e38, 0.0, -0.0, -2.0,
                       np.inf, np.nan, 1e-45, 2.0 ** -126, 7.25])
    for trial in range(4):
        sc = pool[rng.integers(0, pool.size, ns)] if gran != PT else pool[trial * 4:trial * 4 + 1]
        sc = sc * rng.uniform(0.9, 1.1, sc.shape).astype(np.float32) if trial == 3 else sc
        _check(bits, fmt, gran, gs.FP8_SCALE_GIVEN, dev, np.ascontiguousarray(sc, np.float32))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_every_bf16_x_amax_pair(fmt, dev):
    """Every pair of positive finite BF16 values x <= amax, laid out as 1x128
    blocks that each hold one amax and 127 values x (both signs): the codes
    from the reciprocal-and-FMA division equal the oracle's IEEE division
    for the whole input space of BF16 x and block amax."""
    pos = np.arange(1, 0x7F80, dtype=np.uint16)            # positive finite BF16
    blocks_done = 0
    chunk_amax = 4096
    for a0 in range(0, pos.size, chunk_amax):
        amaxes = pos[a0:a0 + chunk_amax]
        rows = []
        for a in amaxes:
            xs = pos[:np.searchsorted(pos, a, side="right")]
            nb = -(-xs.size // 127)
            pad = np.full(nb * 127, a, np.uint16)
            pad[:xs.size] = xs
            blk = np.empty((nb, 128), np.uint16)
            blk[:, 0] = a
            blk[:, 1:] = pad.reshape(nb, 127)
            blk[1::2, 1:] |= 0x8000                       # negative copies in odd blocks
            rows.append(blk)
        x = np.ascontiguousarray(np.concatenate(rows))
        c, s, _, _ = _run(x, fmt, B1, gs.FP8_SCALE_FROM_AMAX, dev)
        rc, rs, _ = oracle.quantize(x, fmt, B1)
        assert np.array_equal(s, rs.view(np.uint32))
        if not np.array_equal(c, rc):
            bad = np.argwhere(c != rc)[:5]
            raise AssertionError("pair mismatch at %s" % [(hex(x[tuple(b)]), hex(x[b[0], 0]))
                                                          for b in bad])
        blocks_done += x.shape[0]
    assert blocks_done > 4_000_000


def test_dequantize_all_codes_all_granularities(dev):
    rng = np.random.default_rng(5)
    for fmt in (E4M3, E5M2):
        for gran, (rows, cols) in ((PT, (16, 16)), (B1, (2, 256)), (B128, (128, 256)),
                                   (B32, (2, 256))):
            codes = np.tile(np.arange(256, dtype=np.uint8), rows * cols // 256).reshape(rows, cols)
            ns = oracle.n_scales(rows, cols, gran)
            for sc in (np.float32([1.0] * ns), rng.uniform(1e-3, 10, ns).astype(np.float32),
                       np.float32([0.0] * ns), np.float32([np.inf] * ns)):
                c = torch.from_numpy(codes).to(dev)
                s = torch.from_numpy(sc).to(dev)
                out = gs.fp8_dequantize(c, fmt, gran, s)
                ref = oracle.dequantize(codes, fmt, gran, sc)
                torch.cuda.synchronize()
                assert np.array_equal(_u32(out), ref.reshape(-1).view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(128, 128), (1152, 384), (256, 5248), (384, 6016),
                                       (640, 3968), (256, 18432)])
def test_dequantize_128x128_tile_lookup(rows, cols, dev):
    """The 128x128 dequantizers walk the codes in row-major order and find
    each group's tile from its position: one row per work item or many
    (narrow matrices), and block counts per row (41 for 5248 columns, 47 for
    6016) where the FP32 quotient needs its one-off correction.  Every tile
    has its own scale, so a wrong tile shows."""
    rng = np.random.default_rng(rows * 7 + cols)
    codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    ns = oracle.n_scales(rows, cols, B128)
    sc = np.ldexp(rng.uniform(1.0, 2.0, ns), rng.integers(-20, 20, ns)).astype(np.float32)
    c = torch.from_numpy(codes).to(dev)
    s = torch.from_numpy(sc).to(dev)
    for fmt in (E4M3, E5M2):
        out = gs.fp8_dequantize(c, fmt, B128, s)
        out16 = gs.fp8_dequantize_bf16(c, fmt, B128, s)
        torch.cuda.synchronize()
        assert np.array_equal(_u32(out), oracle.dequantize(codes, fmt, B128, sc).reshape(-1).view(np.uint32))
        assert np.array_equal(out16.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.dequantize_bf16(codes, fmt, B128, sc))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_matrices(dtype, dev):
    """Empty inputs at every granularity: nothing is written except the
    per-tensor scale, which an empty tensor still gets (the floor scale, as
    the oracle computes it), both formats."""
    for fmt in (E4M3, E5M2):
        for gran, shape in ((PT, (0, 5)), (PT, (7, 0)), (B1, (0, 256)), (B128, (0, 128)),
                            (B128, (128, 0)), (B32, (0, 64))):
            x = torch.empty(shape, dtype=dtype, device=dev)
            codes = torch.empty(shape, dtype=torch.uint8, device=dev)
            ns = oracle.n_scales(*shape, gran)
            sc = torch.full((max(ns, 1),), -1.0, device=dev)
            gs.fp8_quantize(x, fmt, gran, gs.FP8_SCALE_FROM_AMAX, codes, sc)
            out = gs.fp8_dequantize(codes, fmt, gran, sc)
            torch.cuda.synchronize()
            assert out.shape == shape
            if gran == PT:
                _, rs, _ = oracle.quantize(np.zeros(shape, np.float32), fmt, gran)
                assert _u32(sc)[0] == rs.reshape(-1).view(np.uint32)[0]
            else:
                assert float(sc[0].item()) == -1.0


def test_tiny_per_tensor_case(dev):
    """1024x1024 BF16 N(0,1) per-tensor E4M3 and its dequantization."""
    q = synth.tiny_quant()
    bits = synth.as_u16_numpy(synth.to_bf16_tensor(q.gen(torch.arange(q.rows * q.cols))))
    _check(bits.reshape(q.rows, q.cols), q.fmt, q.gran, gs.FP8_SCALE_FROM_AMAX, dev)


def test_abi_shape_and_alignment_errors(dev):
    x = torch.zeros(128, 200, dtype=torch.bfloat16, device=dev)
    with pytest.raises(gs.GSError) as e:
        gs.fp8_quantize(x, E4M3, B1)
    assert e.value.status == -3
    y = torch.zeros(4 * 128 + 1, dtype=torch.bfloat16, device=dev)[1:].view(4, 128)
    with pytest.raises(gs.GSError) as e:
        gs.fp8_quantize(y, E4M3, B1)                     # 16-byte alignment required
    assert e.value.status == -6


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_every_fp32_value_given_scale_one(fmt, dev):
    """All 2^32 FP32 bit patterns through the per-tensor given-scale cast with
    s = 1 (y = x exactly): the codes equal the oracle's for the whole FP32
    input space, NaN, Inf, subnormals and saturation included."""
    chunk = 1 << 28
    sc = torch.ones(1, dtype=torch.float32, device=dev)
    codes = torch.empty((1, chunk), dtype=torch.uint8, device=dev)
    for lo in range(0, 1 << 32, chunk):
        host = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        x = torch.from_numpy(host).to(dev).view(1, chunk)
        gs.fp8_quantize(x, fmt, PT, gs.FP8_SCALE_GIVEN, codes=codes, scales=sc)
        got = codes.cpu().numpy().reshape(-1)
        ref = oracle.cast(host, 1.0, fmt)
        if not np.array_equal(got, ref):
            bad = np.flatnonzero(got != ref)[:5]
            raise AssertionError("fp32 patterns %s: gpu %s oracle %s" % (
                [hex(lo + int(i)) for i in bad], got[bad].tolist(), ref[bad].tolist()))


def _fp32_midpoint_matrix(rng, rows, cols, fmt, br, bc):
    """FP32 [rows, cols] whose br x bc blocks each hold one +-A (a random
    non-power-of-two amax, exponents -40..40) and elsewhere values within
    +-8 ulps of x = fl32(m * s) for random midpoints m between adjacent FP8
    values, with s = fl32(max(A, fl32(1e-12)) / MAX) that block's scale, so
    that the quotients x / s straddle the FP8 rounding boundaries."""
    vals = np.unique(np.abs(oracle.fp8_decode_table(fmt)[np.isfinite(oracle.fp8_decode_table(fmt))]))
    mids = (vals[:-1] + vals[1:]) / 2
    nbr, nbc = rows // br, cols // bc
    mant = rng.integers(1, 1 << 23, size=(nbr, nbc)).astype(np.uint32)
    expo = rng.integers(127 - 40, 127 + 41, size=(nbr, nbc)).astype(np.uint32)
    A = ((expo << 23) | mant).view(np.float32)
    s = np.maximum(A, np.float32(1e-12)) / np.float32(oracle.FMT_MAX[fmt])
    s_full = np.repeat(np.repeat(s, br, 0), bc, 1)
    A_full = np.repeat(np.repeat(A, br, 0), bc, 1)
    m = mids[rng.integers(0, mids.size, size=(rows, cols))]
    x0 = (m * s_full.astype(np.float64)).astype(np.float32)
    x = (x0.view(np.uint32).astype(np.int64) + rng.integers(-8, 9, size=(rows, cols)))
    x = np.minimum(x.astype(np.uint32).view(np.float32), A_full)
    x = np.where(rng.integers(0, 2, size=(rows, cols)) == 1, -x, x).astype(np.float32)
    for bi in range(nbr):                         # one +-A per block: its amax
        for bj in range(nbc):
            r, c = bi * br + rng.integers(0, br), bj * bc + rng.integers(0, bc)
            x[r, c] = A[bi, bj] if rng.integers(0, 2) else -A[bi, bj]
    return x


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp32_midpoints_with_non_power_of_two_scales(fmt, dev):
    """FP32 input in amax mode at every granularity: quotients within +-8
    ulps of FP8 midpoints under non-power-of-two block scales, where a
    division that is off in the last bit would change the code; codes,
    scales and dequantized values against the oracle."""
    rng = np.random.default_rng(2900 + fmt)
    for gran, (rows, cols), (br, bc) in ((B1, (512, 1024), (1, 128)),
                                         (B128, (512, 1024), (128, 128)),
                                         (B32, (256, 1024), (1, 32)),
                                         (PT, (512, 1024), (512, 1024))):
        x = _fp32_midpoint_matrix(rng, rows, cols, fmt, br, bc)
        _check(x, fmt, gran, gs.FP8_SCALE_FROM_AMAX, dev)


def _degenerate_bf16(rng, rows, cols, block_rows, block_cols):
    """BF16 bit patterns where every block (block_rows x block_cols) is one
    degenerate kind: all +0, all -0, all NaN, all +-Inf, NaN and Inf mixed,
    all BF16 subnormals (amax below the 1e-12 floor times MAX), one huge
    finite value among zeros, one value among NaNs, or ordinary N(0,1)."""
    bits = np.zeros((rows, cols), np.uint16)
    kinds = 9
    for bi, r0 in enumerate(range(0, rows, block_rows)):
        for bj, c0 in enumerate(range(0, cols, block_cols)):
            b = bits[r0:r0 + block_rows, c0:c0 + block_cols]
            kind = (bi * 7 + bj) % kinds
            if kind == 1:
                b[:] = 0x8000
            elif kind == 2:
                b[:] = 0x7FC0 | rng.integers(0, 0x40, b.shape).astype(np.uint16)
            elif kind == 3:
                b[:] = np.where(rng.random(b.shape) < 0.5, 0x7F80, 0xFF80)
            elif kind == 4:
                b[:] = np.where(rng.random(b.shape) < 0.5, 0x7FC1, 0xFF80)
            elif kind == 5:
                b[:] = rng.integers(1, 0x80, b.shape).astype(np.uint16) | \
                    (rng.integers(0, 2, b.shape).astype(np.uint16) << 15)
            elif kind == 6:
                b.reshape(-1)[int(rng.integers(0, b.size))] = 0x7F7F       # the largest BF16
            elif kind == 7:
                b[:] = 0xFFC0
                b.reshape(-1)[int(rng.integers(0, b.size))] = 0x3F80       # 1.0 among NaNs
            elif kind == 8:
                x = rng.standard_normal(b.shape).astype(np.float32)
                b[:] = (x.view(np.uint32) >> 16).astype(np.uint16)
    return bits


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_blocks_every_granularity(fmt, dtype, dev):
    """Blocks that are entirely zero, NaN, Inf, subnormal, or a lone value
    among zeros or NaNs, laid out on each granularity's own block grid
    (and, for per-tensor, whole matrices of each kind), against the oracle:
    the finite-only amax, the 1e-12 floor, saturation, NaN codes and the
    MX power-of-two scale on every degenerate case."""
    rng = np.random.default_rng(4242 + fmt + 2 * (dtype == "f32"))

    def conv(bits):
        x = bits if dtype == "bf16" else (bits.astype(np.uint32) << 16).view(np.float32)
        return np.ascontiguousarray(x)

    rows, cols = 384, 640
    for gran, (br, bc) in ((B1, (1, 128)), (B32, (1, 32)), (B128, (128, 128))):
        _check(conv(_degenerate_bf16(rng, rows, cols, br, bc)), fmt, gran,
               gs.FP8_SCALE_FROM_AMAX, dev)
    xmx = conv(_degenerate_bf16(rng, 96, 320, 1, 32))
    xt = torch.from_numpy(xmx.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
        else torch.from_numpy(xmx)
    x = xt.to(dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    codes, sc = gs.fp8_quantize_mx(x, fmt, nonfinite=nf)
    deq = gs.fp8_dequantize_mx(codes, fmt, sc)
    rc, rs, rnf = oracle.quantize_mx(xmx, fmt)
    rd = oracle.dequantize_mx(rc, fmt, rs)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), rc), "MX codes"
    assert np.array_equal(sc.cpu().numpy(), rs), "MX scale bytes"
    assert np.array_equal(_u32(deq), rd.reshape(-1).view(np.uint32)), "MX dequantized values"
    assert int(nf.item()) == rnf
    # per-tensor: a whole matrix of each kind (a ragged 77 x 93 one)
    for kind_rows in range(9):
        bits = _degenerate_bf16(rng, 77, 93, 77, 93)
        if kind_rows:
            bits = _degenerate_bf16(np.random.default_rng(kind_rows), 77 * 9, 93, 77, 93)
            bits = np.ascontiguousarray(bits[77 * kind_rows:77 * (kind_rows + 1)])
        _check(conv(bits), fmt, PT, gs.FP8_SCALE_FROM_AMAX, dev)
