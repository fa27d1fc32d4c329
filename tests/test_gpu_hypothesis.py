"""GPU parity driven by hypothesis (derandomized, no example database):
gradient lists of random length with sizes around the 2048-element chunk
edges (0, 1, 7, 2047-2049, 4095-4097, up to 20000), views misaligned by up to
7 elements, and random scales, through the unscale and the unscale + exact
sum of squares; and random legal shapes of every quantize granularity (MX
included), both formats, BF16 and FP32, with planted special values.  Every
example is compared with the oracle bit for bit."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import loss_scaling_fp8_amd as gs
import oracle

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))
DEV = torch.device("cuda:0")
M64 = (1 << 64) - 1


def _u32(t):
    return t.detach().cpu().contiguous().numpy().reshape(-1).view(np.uint32)


sizes = st.one_of(st.sampled_from([0, 1, 7, 2047, 2048, 2049, 4095, 4096, 4097]),
                  st.integers(0, 20000))
scales = st.one_of(st.integers(-24, 30).map(lambda k: float(np.ldexp(np.float32(1), k))),
                   st.floats(0.01, 1e5).map(lambda v: float(np.float32(v))))


@SETTINGS
@given(st.lists(st.tuples(sizes, st.integers(0, 7), st.integers(0, 7)), max_size=6), scales,
       st.integers(0, 2 ** 32 - 1), st.booleans())
def test_unscale_lists(spec, S, seed, with_sumsq):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    rng = np.random.default_rng(seed)
    total = sum(n + 16 for n, _, _ in spec) + 16
    pool = torch.empty(total, dtype=torch.float16, device=DEV)
    opool = torch.empty(total, dtype=torch.float32, device=DEV)
    host, grads, outs, off = [], [], [], 0
    for n, a, b in spec:
        h = rng.integers(0, 0x10000, size=n, dtype=np.uint32).astype(np.uint16)
        g = pool[off + a: off + a + n]
        if n:
            g.copy_(torch.from_numpy(h.view(np.int16)).view(torch.float16).to(DEV))
        host.append(h)
        grads.append(g)
        outs.append(opool[off + b: off + b + n])
        off += n + 16
    Sd = torch.tensor([S], dtype=torch.float32, device=DEV)
    f = torch.zeros(1, dtype=torch.int32, device=DEV)
    if with_sumsq:
        acc = torch.zeros(2, dtype=torch.int64, device=DEV)
        ns = torch.zeros(1, dtype=torch.float64, device=DEV)
        gs.gs_unscale_check_sumsq(grads, outs, Sd, f, acc, ns)
        ref, rflag, racc, rns = oracle.unscale_check_sumsq(host, S)
    else:
        gs.gs_unscale_check(grads, outs, Sd, f)
        ref, rflag = oracle.unscale_check(host, S)
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert np.array_equal(_u32(o), r.view(np.uint32))
    assert int(f.item()) == rflag
    if with_sumsq:
        assert tuple(int(v) & M64 for v in acc.cpu().tolist()) == tuple(racc)
        assert np.float64(ns.item()).view(np.uint64) == np.float64(rns).view(np.uint64)


@st.composite
def quant_case(draw):
    gran = draw(st.sampled_from(["pt", "1x128", "128x128", "1x32", "mx"]))
    if gran == "pt":
        rows, cols = draw(st.integers(1, 500)), draw(st.integers(1, 700))
    elif gran == "1x128":
        rows, cols = draw(st.integers(1, 300)), 128 * draw(st.integers(1, 6))
    elif gran == "128x128":
        rows, cols = 128 * draw(st.integers(1, 3)), 128 * draw(st.integers(1, 4))
    else:
        rows, cols = draw(st.integers(1, 300)), 32 * draw(st.integers(1, 20))
    return gran, rows, cols, draw(st.integers(0, 1)), draw(st.sampled_from(["bf16", "f32"])), \
        draw(st.integers(0, 2 ** 32 - 1))


GRAN = {"pt": gs.FP8_PER_TENSOR, "1x128": gs.FP8_BLOCK_1x128, "128x128": gs.FP8_BLOCK_128x128,
        "1x32": gs.FP8_BLOCK_1x32}


@SETTINGS
@given(quant_case())
def test_quantize_shapes(case):
    gran, rows, cols, fmt, dtype, seed = case
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.ldexp(np.float32(1.0), rng.integers(-20, 21, (rows, 1))).astype(np.float32)
    flat = x.reshape(-1)
    pos = rng.choice(flat.size, size=max(1, flat.size // 200), replace=False)
    flat[pos] = rng.choice(np.float32([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-41, 500.0, 6e4]),
                           size=pos.size)
    if dtype == "bf16":
        b = x.view(np.uint32)
        xh = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
        xh[np.isnan(x)] = 0x7FC0
        xd = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        xh = x
        xd = torch.from_numpy(x).to(DEV)
    nf = torch.zeros(1, dtype=torch.int32, device=DEV)
    if gran == "mx":
        codes, sc = gs.fp8_quantize_mx(xd, fmt, nonfinite=nf)
        rc, rs, rnf = oracle.quantize_mx(xh, fmt)
        torch.cuda.synchronize()
        assert np.array_equal(sc.cpu().numpy(), rs)
    else:
        codes, sc = gs.fp8_quantize(xd, fmt, GRAN[gran], nonfinite=nf)
        rc, rs, rnf = oracle.quantize(xh, fmt, GRAN[gran])
        torch.cuda.synchronize()
        assert np.array_equal(_u32(sc), rs.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert int(nf.item()) == rnf
