"""GPU parity on seeded random cases, through the C ABI against the oracle,
bit for bit: quantize/dequantize at random legal shapes of every granularity
(MX included), both formats, BF16 and FP32 inputs, amax-derived and given
scales, with row-varying magnitudes over 60 binades and planted special
values; and the unscale + exact sum of squares on random gradient lists
(sizes, base offsets, scales, running totals)."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle

pytestmark = pytest.mark.gpu

PT, B1, B128, B32 = gs.FP8_PER_TENSOR, gs.FP8_BLOCK_1x128, gs.FP8_BLOCK_128x128, gs.FP8_BLOCK_1x32
MX = "mx"
M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _u32(t):
    return t.detach().cpu().contiguous().numpy().reshape(-1).view(np.uint32)


def _shape(rng, gran):
    if gran == PT:
        return int(rng.integers(1, 700)), int(rng.integers(1, 900))
    if gran == B128:
        return 128 * int(rng.integers(1, 4)), 128 * int(rng.integers(1, 5))
    if gran == B1:
        return int(rng.integers(1, 300)), 128 * int(rng.integers(1, 7))
    return int(rng.integers(1, 300)), 32 * int(rng.integers(1, 21))      # 1x32 and MX


def _data(rng, rows, cols, dtype):
    """FP32 values N(0,1) times 2^k per row (k in [-30, 30]), 1% special
    values (NaN, +-Inf, +-0, FP32/BF16 subnormals); BF16 as rounded bits."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.ldexp(np.float32(1.0), rng.integers(-30, 31, (rows, 1))).astype(np.float32)
    flat = x.reshape(-1)
    k = max(1, flat.size // 100)
    pos = rng.choice(flat.size, size=min(k, flat.size), replace=False)
    flat[pos] = rng.choice(np.float32([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-40, -3e-39, 1e-30]),
                           size=pos.size)
    if dtype == "f32":
        return x
    b = x.view(np.uint32)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)      # RNE to BF16
    r[np.isnan(x.reshape(rows, cols))] = 0x7FC0
    return r


def _to_dev(xh, dev):
    if xh.dtype == np.uint16:
        return torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(xh).to(dev)


@pytest.mark.parametrize("seed", range(4))
def test_random_quantize_cases(dev, seed):
    rng = np.random.default_rng(9000 + seed)
    for trial in range(12):
        gran = [PT, B1, B128, B32, MX][int(rng.integers(0, 5))]
        fmt = int(rng.integers(0, 2))
        dtype = ["bf16", "f32"][int(rng.integers(0, 2))]
        rows, cols = _shape(rng, gran)
        xh = np.ascontiguousarray(_data(rng, rows, cols, dtype))
        x = _to_dev(xh, dev)
        tag = (seed, trial, gran, fmt, dtype, rows, cols)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        if gran == MX:
            codes, sc = gs.fp8_quantize_mx(x, fmt, nonfinite=nf)
            deq = gs.fp8_dequantize_mx(codes, fmt, sc)
            rc, rs, rnf = oracle.quantize_mx(xh, fmt)
            rd = oracle.dequantize_mx(rc, fmt, rs)
            torch.cuda.synchronize()
            assert np.array_equal(sc.cpu().numpy(), rs), tag
        else:
            given = bool(rng.integers(0, 2))
            mode = gs.FP8_SCALE_GIVEN if given else gs.FP8_SCALE_FROM_AMAX
            scales_h = None
            if given:
                ns = oracle.n_scales(rows, cols, gran)
                scales_h = np.ldexp(np.float32(1.0), rng.integers(-40, 40, ns)).astype(np.float32)
                scales_h *= rng.uniform(0.5, 2.0, ns).astype(np.float32)
                scales_h[rng.random(ns) < 0.05] = np.float32(0.0)
            sc_d = None if scales_h is None else torch.from_numpy(scales_h).to(dev).reshape(
                gs.scale_shape(rows, cols, gran))
            codes, sc = gs.fp8_quantize(x, fmt, gran, mode, scales=sc_d, nonfinite=nf)
            deq = gs.fp8_dequantize(codes, fmt, gran, sc)
            rc, rs, rnf = oracle.quantize(xh, fmt, gran, mode, scales_h)
            rd = oracle.dequantize(rc, fmt, gran, rs)
            torch.cuda.synchronize()
            assert np.array_equal(_u32(sc), rs.view(np.uint32)), tag
        c = codes.cpu().numpy()
        if not np.array_equal(c, rc):
            bad = np.argwhere(c != rc)[:4]
            raise AssertionError("codes differ %s at %s" % (tag, bad.tolist()))
        assert np.array_equal(_u32(deq), rd.reshape(-1).view(np.uint32)), tag
        assert int(nf.item()) == rnf, tag


@pytest.mark.parametrize("seed", range(3))
def test_random_unscale_sumsq_lists(dev, seed):
    rng = np.random.default_rng(9100 + seed)
    pool = torch.empty(1 << 21, dtype=torch.float16, device=dev)
    opool = torch.empty(1 << 21, dtype=torch.float32, device=dev)
    for trial in range(10):
        m = int(rng.integers(1, 12))
        host, grads, outs = [], [], []
        off = 0
        for k in range(m):
            n = int(rng.choice([0, rng.integers(1, 64), rng.integers(1, 5000), rng.integers(1, 150000)]))
            h = rng.integers(0, 0x10000, size=n, dtype=np.uint32).astype(np.uint16)
            sh_in, sh_out = int(rng.integers(0, 8)), int(rng.integers(0, 8))
            host.append(h)
            g = pool[off + sh_in: off + sh_in + n]
            if n:
                g.copy_(torch.from_numpy(h.view(np.int16)).view(torch.float16).to(dev))
            grads.append(g)
            outs.append(opool[off + sh_out: off + sh_out + n])
            off += n + 16
        S = float(rng.choice([2.0 ** int(rng.integers(-20, 30)), float(rng.uniform(0.1, 1e6))]))
        start = (int(rng.integers(0, 1 << 63)) * 2 % (1 << 64), int(rng.integers(0, 1 << 40)))
        Sd = torch.tensor([S], dtype=torch.float32, device=dev)
        f = torch.zeros(1, dtype=torch.int32, device=dev)
        acc = torch.tensor([start[0] - (1 << 64) if start[0] >= (1 << 63) else start[0], start[1]],
                           dtype=torch.int64, device=dev)
        ns = torch.zeros(1, dtype=torch.float64, device=dev)
        gs.gs_unscale_check_sumsq(grads, outs, Sd, f, acc, ns)
        ref, rflag, racc, rns = oracle.unscale_check_sumsq(host, S, sumsq=start)
        torch.cuda.synchronize()
        tag = (seed, trial, m, S)
        for o, r in zip(outs, ref):
            assert np.array_equal(_u32(o), r.view(np.uint32)), tag
        assert int(f.item()) == rflag, tag
        lo, hi = (int(v) & M64 for v in acc.cpu().tolist())
        assert (lo, hi) == tuple(racc), tag
        assert np.float64(ns.item()).view(np.uint64) == np.float64(rns).view(np.uint64), tag
