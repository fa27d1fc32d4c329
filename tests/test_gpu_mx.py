"""GPU parity: MX-style 1x32 quantize / dequantize with E8M0 power-of-two
scales (fp8_quantize_mx / fp8_dequantize_mx) through the C ABI, bit for bit
against the oracle (codes, scale bytes, dequantized FP32, nonfinite flag)."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
from test_gpu_quant import _special_bf16, _u32

pytestmark = pytest.mark.gpu

E4M3, E5M2 = gs.FP8_E4M3, gs.FP8_E5M2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _to_dev(x_host, dev):
    if x_host.dtype == np.uint16:
        return torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x_host).to(dev)


def _check(x_host, fmt, dev):
    x = _to_dev(np.ascontiguousarray(x_host), dev)
    nf = torch.zeros(1, dtype=torch.int32, device=dev)
    codes, sc = gs.fp8_quantize_mx(x, fmt, nonfinite=nf)
    deq = gs.fp8_dequantize_mx(codes, fmt, sc)
    torch.cuda.synchronize()
    rc, rs, rnf = oracle.quantize_mx(x_host, fmt)
    rd = oracle.dequantize_mx(rc, fmt, rs)
    c = codes.cpu().numpy()
    if not np.array_equal(c, rc):
        bad = np.argwhere(c != rc)[:5]
        raise AssertionError("codes differ at %s" % bad.tolist())
    assert np.array_equal(sc.cpu().numpy(), rs), "scale bytes differ"
    assert np.array_equal(_u32(deq), rd.reshape(-1).view(np.uint32)), "dequantized values differ"
    assert int(nf.item()) == rnf


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_special_values_all_shapes(fmt, dtype, dev):
    rng = np.random.default_rng(500 + fmt)
    for rows, cols in [(1, 32), (3, 96), (130, 256), (257, 608), (1024, 1024)]:
        bits = _special_bf16(rng, rows, cols)
        x = bits if dtype == "bf16" else (bits.astype(np.uint32) << 16).view(np.float32)
        _check(x, fmt, dev)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_bf16_x_amax_pairs_every_37th_amax(fmt, dev):
    """Positive finite BF16 x <= amax for every 37th amax, as 1x32 blocks
    holding one amax and 31 values x (negative copies in odd blocks)."""
    pos = np.arange(1, 0x7F80, dtype=np.uint16)
    rows = []
    for a in pos[::37]:
        xs = pos[:np.searchsorted(pos, a, side="right")]
        nb = -(-xs.size // 31)
        pad = np.full(nb * 31, a, np.uint16)
        pad[:xs.size] = xs
        blk = np.empty((nb, 32), np.uint16)
        blk[:, 0] = a
        blk[:, 1:] = pad.reshape(nb, 31)
        blk[1::2, 1:] |= 0x8000
        rows.append(blk)
    x = np.concatenate(rows)
    x = x[: x.shape[0] // 8 * 8].reshape(-1, 256)        # 8 blocks per row
    _check(x, fmt, dev)
    assert x.size > 10_000_000


def test_dequantize_all_codes_extreme_bytes(dev):
    codes = np.tile(np.arange(256, dtype=np.uint8)[None, :], (8, 1))
    for fmt in (E4M3, E5M2):
        for bytes_ in ([0, 1, 126, 127, 128, 200, 254, 255], [255] * 8, [0] * 8):
            sc = np.repeat(np.uint8(bytes_)[:, None], 8, axis=1)        # [8 rows][8 blocks]
            out = gs.fp8_dequantize_mx(torch.from_numpy(codes).to(dev), fmt,
                                       torch.from_numpy(sc).to(dev))
            ref = oracle.dequantize_mx(codes, fmt, sc)
            torch.cuda.synchronize()
            assert np.array_equal(_u32(out), ref.reshape(-1).view(np.uint32)), (fmt, bytes_)


def test_agrees_with_fp32_scaled_1x32_where_scale_is_a_power_of_two(dev):
    """Blocks whose amax is MAX * 2^k (k >= -8, so the planted value is the
    block max over the uniform(-1, 1) rest): the FP32 block scale is already
    a power of two, so MX codes equal the 1x32 FP32-scale codes."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (64, 256)).astype(np.float32)
    x[:, ::32] = np.float32(448.0) * np.ldexp(1.0, rng.integers(-8, 20, (64, 8))).astype(np.float32)
    xd = torch.from_numpy(x).to(dev)
    c_mx, s_mx = gs.fp8_quantize_mx(xd, E4M3)
    c_32, s_32 = gs.fp8_quantize(xd, E4M3, gs.FP8_BLOCK_1x32)
    torch.cuda.synchronize()
    assert torch.equal(c_mx, c_32)
    assert np.array_equal(s_mx.cpu().numpy(), (_u32(s_32) >> 23).astype(np.uint8).reshape(64, 8))


def test_abi_errors(dev):
    x = torch.zeros(4, 48, dtype=torch.bfloat16, device=dev)
    with pytest.raises(gs.GSError) as e:
        gs.fp8_quantize_mx(x, E4M3)
    assert e.value.status == -3
    with pytest.raises(gs.GSError) as e:
        gs.fp8_quantize_mx(torch.zeros(4, 64, dtype=torch.bfloat16, device=dev), 7)
    assert e.value.status == -5
    with pytest.raises(TypeError):
        gs.fp8_quantize_mx(torch.zeros(4, 64, dtype=torch.float16, device=dev), E4M3)
