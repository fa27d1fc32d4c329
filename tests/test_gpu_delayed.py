"""GPU parity: delayed per-tensor scaling through the C ABI, step by step
against the oracle (codes, the scale used, the history ring, its position,
the next scale, the nonfinite flag)."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _u32(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32).reshape(-1)


def _steps(rng, shape, nsteps):
    """A sequence of tensors: steady N(0, 3^2) steps, one spike x300, one
    with NaN and Inf, one all-zero."""
    xs = []
    for t in range(nsteps):
        x = (rng.standard_normal(shape) * 3).astype(np.float32)
        if t == 4:
            x.reshape(-1)[rng.integers(0, x.size, 7)] *= 300.0
        if t == 6:
            x.reshape(-1)[rng.integers(0, x.size, 5)] = np.nan
            x.reshape(-1)[rng.integers(0, x.size, 3)] = -np.inf
        if t == 8:
            x[:] = 0.0
        xs.append(x)
    return xs


@pytest.mark.parametrize("fmt", [gs.FP8_E4M3, gs.FP8_E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hlen", [1, 4, 16])
def test_delayed_sequence_matches_oracle(fmt, dtype, hlen, dev):
    rng = np.random.default_rng(100 * hlen + 10 * fmt + (dtype == "bf16"))
    shape = (333, 517)                      # ragged: not a multiple of the vector width
    R = oracle.DelayedState(hlen, init_scale=0.75)
    st = torch.tensor([0.75], dtype=torch.float32, device=dev)
    hist = torch.zeros(hlen, dtype=torch.float32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    for t, xf in enumerate(_steps(rng, shape, 11)):
        if dtype == "bf16":
            bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
            x_host = bits
            x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            x_host = xf
            x = torch.from_numpy(xf).to(dev)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        codes, used = gs.fp8_quantize_delayed(x, fmt, st, hist, pos, nonfinite=nf)
        rc, rused, rnf = oracle.quantize_delayed(x_host, fmt, R)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc), (t, "codes")
        assert _u32(used)[0] == np.float32(rused).view(np.uint32), (t, "scale used")
        assert np.array_equal(_u32(hist), R.history.view(np.uint32)), (t, "history")
        assert int(pos.item()) == int(R.pos[0]), (t, "pos")
        assert _u32(st)[0] == R.scale.view(np.uint32)[0], (t, "next scale")
        assert int(nf.item()) == rnf, (t, "nonfinite")


def test_delayed_large_and_empty(dev):
    """A 8192x8192 tensor (the grid uses every partial slot) and an empty
    one (only the history moves)."""
    rng = np.random.default_rng(7)
    R = oracle.DelayedState(4, init_scale=2.0)
    st = torch.tensor([2.0], dtype=torch.float32, device=dev)
    hist = torch.zeros(4, dtype=torch.float32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    for x_host in [(rng.standard_normal((8192, 8192)) * 5).astype(np.float32),
                   np.zeros((0, 7), np.float32),
                   (rng.standard_normal((8192, 8192))).astype(np.float32)]:
        x = torch.from_numpy(x_host).to(dev)
        codes, used = gs.fp8_quantize_delayed(x, gs.FP8_E4M3, st, hist, pos)
        rc, rused, _ = oracle.quantize_delayed(x_host, gs.FP8_E4M3, R)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert _u32(used)[0] == np.float32(rused).view(np.uint32)
        assert np.array_equal(_u32(hist), R.history.view(np.uint32))
        assert _u32(st)[0] == R.scale.view(np.uint32)[0]


def test_delayed_longest_history(dev):
    """The largest history the ABI accepts (1024 entries, one per lane of
    the update workgroup), with the ring position already past the first
    wrap, and one entry past the limit refused."""
    hlen = 1024
    rng = np.random.default_rng(1024)
    R = oracle.DelayedState(hlen, init_scale=0.5)
    R.pos[0] = 2 * hlen - 3                  # reduced modulo the length
    st = torch.tensor([0.5], dtype=torch.float32, device=dev)
    hist = torch.zeros(hlen, dtype=torch.float32, device=dev)
    pos = torch.tensor([2 * hlen - 3], dtype=torch.int32, device=dev)
    for t, xf in enumerate(_steps(rng, (96, 160), 11)):
        x = torch.from_numpy(xf).to(dev)
        codes, used = gs.fp8_quantize_delayed(x, gs.FP8_E4M3, st, hist, pos)
        rc, rused, _ = oracle.quantize_delayed(xf, gs.FP8_E4M3, R)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc), (t, "codes")
        assert _u32(used)[0] == np.float32(rused).view(np.uint32), (t, "scale used")
        assert np.array_equal(_u32(hist), R.history.view(np.uint32)), (t, "history")
        assert int(pos.item()) == int(R.pos[0]), (t, "pos")
        assert _u32(st)[0] == R.scale.view(np.uint32)[0], (t, "next scale")
    big = torch.zeros(hlen + 1, dtype=torch.float32, device=dev)
    with pytest.raises(gs.GSError):
        gs.fp8_quantize_delayed(x, gs.FP8_E4M3, st, big, pos)
