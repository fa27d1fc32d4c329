"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times: sampled outputs checked one by one against the oracle, plus
properties that hold at any size.

Workloads (seeded, synthetic; see synth/):
  * Llama-3-8B-shaped FP16 gradient set, 291 tensors / 8,030,261,248
    elements, S = 2^15, 10 steps with an Inf in lm_head at step 2;
  * DeepSeek-V3-shaped BF16 activations 16384x7168 (1x128) and weights
    7168x18432 (128x128), E4M3;
  * 8192x8192 per-tensor E4M3 (0.1% x1000 outliers) and E5M2 (Laplace);
  * four 16384x32768 special-value tensors, every granularity, both
    formats, both scale modes.
"""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu

PT, B1, B128 = gs.FP8_PER_TENSOR, gs.FP8_BLOCK_1x128, gs.FP8_BLOCK_128x128


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _u32(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy().view(np.uint32).reshape(-1)


def test_generators_identical_on_cpu_and_gpu(dev):
    """The seeded generators give the same bits on both devices, so the
    oracle can regenerate any sample of a tensor built on the GPU."""
    idx = torch.arange(0, 1 << 20, 997, dtype=torch.int64)
    specs = synth.deepseek_v3_blocks() + synth.per_tensor_at_scale() + synth.special_values_4gib()
    for sp in specs:
        assert torch.equal(sp.gen(idx), sp.gen(idx.to(dev)).cpu()), sp.name
    g = synth.llama3_8b_gradset()
    for t in (0, 5, 290):
        assert torch.equal(g.gen(t, idx), g.gen(t, idx.to(dev)).cpu())


def test_llama3_8b_gradset_10_steps(dev):
    g = synth.llama3_8b_gradset()
    grads = [g.full(t, dev) for t in range(len(g.tensors))]
    outs = [torch.empty(sp.numel, dtype=torch.float32, device=dev) for sp in g.tensors]
    S = torch.tensor([g.scale], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    skips = torch.zeros(1, dtype=torch.int64, device=dev)
    R = oracle.ScalerState(g.scale)
    rng = np.random.default_rng(44)
    inj_t, inj_i, inj_bits = g.injections[2][0]
    inj_orig = int(g.gen(inj_t, torch.tensor([inj_i]))[0])
    for step in range(1, g.steps + 1):
        if step == 2:
            grads[inj_t][inj_i:inj_i + 1].fill_(float("inf"))
        gs.gs_unscale_check(grads, outs, S, found)
        # samples: random elements of every tensor, both ends of each, the injection
        S_before = float(R.S)
        for t, sp in enumerate(g.tensors):
            n = sp.numel
            k = max(8, min(4096, n // 100000))
            idx = np.unique(np.concatenate([rng.integers(0, n, k), np.arange(min(8, n)),
                                            np.arange(max(0, n - 8), n)]))
            if t == inj_t:
                idx = np.unique(np.append(idx, inj_i))
            ti = torch.from_numpy(idx)
            bits = g.gen(t, ti).numpy().astype(np.uint16)
            if step == 2 and t == inj_t:
                bits[np.searchsorted(idx, inj_i)] = inj_bits
            ref, _ = oracle.unscale_check([bits], S_before)
            got = outs[t][ti.to(dev)]
            assert np.array_equal(_u32(got), ref[0].view(np.uint32)), (step, t)
        # property over every element: non-finite outputs exactly where injected
        finite = torch.stack([torch.isfinite(o).all() for o in outs]).all().item()
        assert finite == (step != 2)
        assert int(found.item()) == (1 if step == 2 else 0)
        R.found_inf.value = int(found.item())
        gs.gs_update_scale(S, tracker, found, 2.0, 0.5, 2000, skips)
        oracle.update_scale(R, 2.0, 0.5, 2000)
        torch.cuda.synchronize()
        assert (float(S.item()), int(tracker.item()), int(skips.item())) == \
            (float(R.S), R.tracker.value, R.skips.value)
        if step == 2:
            grads[inj_t][inj_i:inj_i + 1].fill_(float(np.uint16(inj_orig).view(np.float16)))
    assert (float(R.S), R.tracker.value, R.skips.value) == (2.0 ** 14, 8, 1)


def _check_blocks(x_spec, codes, scales, deq, gran, fmt, rng, nsample):
    """Sampled blocks of device tensors codes/scales/deq against the oracle
    run on the same block regenerated on the host; returns the number of
    blocks checked."""
    rows, cols = x_spec.rows, x_spec.cols
    checked = 0
    if gran == B1:
        nb = rows * (cols // 128)
        blocks = np.unique(np.concatenate([rng.integers(0, nb, nsample), [0, nb - 1]]))
        for b in blocks:
            r, j = divmod(int(b), cols // 128)
            idx = torch.arange(r * cols + j * 128, r * cols + j * 128 + 128)
            xb = x_spec.gen(idx).numpy().astype(np.uint16).reshape(1, 128)
            rc, rs, _ = oracle.quantize(xb, fmt, PT)
            sl = (slice(r, r + 1), slice(j * 128, (j + 1) * 128))
            assert np.array_equal(codes[sl].cpu().numpy(), rc), b
            assert _u32(scales[r, j:j + 1])[0] == rs.view(np.uint32)[0], b
            rd = oracle.dequantize(rc, fmt, PT, rs)
            assert np.array_equal(_u32(deq[sl]).reshape(-1), rd.reshape(-1).view(np.uint32)), b
            checked += 1
    else:
        tpr = cols // 128
        nt = (rows // 128) * tpr
        tiles = np.unique(np.concatenate([rng.integers(0, nt, nsample), [0, nt - 1]]))
        for t in tiles:
            ti, tj = divmod(int(t), tpr)
            r = torch.arange(ti * 128, ti * 128 + 128)[:, None]
            c = torch.arange(tj * 128, tj * 128 + 128)[None, :]
            xb = x_spec.gen((r * cols + c).reshape(-1)).numpy().astype(np.uint16).reshape(128, 128)
            rc, rs, _ = oracle.quantize(xb, fmt, PT)
            sl = (slice(ti * 128, ti * 128 + 128), slice(tj * 128, tj * 128 + 128))
            assert np.array_equal(codes[sl].cpu().numpy(), rc), t
            assert _u32(scales[ti, tj:tj + 1])[0] == rs.view(np.uint32)[0], t
            rd = oracle.dequantize(rc, fmt, PT, rs)
            assert np.array_equal(_u32(deq[sl]).reshape(-1), rd.reshape(-1).view(np.uint32)), t
            checked += 1
    return checked


def test_deepseek_v3_block_shapes(dev):
    rng = np.random.default_rng(33)
    for sp in synth.deepseek_v3_blocks():
        x = sp.full(dev)
        nf = torch.zeros(1, dtype=torch.int32, device=dev)
        codes, scales = gs.fp8_quantize(x, sp.fmt, sp.gran, nonfinite=nf)
        deq = gs.fp8_dequantize(codes, sp.fmt, sp.gran, scales)
        torch.cuda.synchronize()
        # properties at full size: finite positive scales, no NaN codes, no flag
        assert torch.isfinite(scales).all() and (scales > 0).all()
        assert not ((codes & 0x7F) == 0x7F).any()
        assert int(nf.item()) == 0
        assert tuple(scales.shape) == gs.scale_shape(sp.rows, sp.cols, sp.gran)
        n = _check_blocks(sp, codes, scales, deq, sp.gran, sp.fmt, rng,
                          3000 if sp.gran == B1 else 40)
        assert n >= (2500 if sp.gran == B1 else 35)


def test_per_tensor_at_scale_full_compare(dev):
    """8192x8192 per-tensor: the whole tensor against the oracle (the input
    bits are the generator's, produced on the GPU and checked identical to
    the CPU generator above)."""
    for sp in synth.per_tensor_at_scale():
        x = sp.full(dev)
        codes, scales = gs.fp8_quantize(x, sp.fmt, PT)
        deq = gs.fp8_dequantize(codes, sp.fmt, PT, scales)
        torch.cuda.synchronize()
        xh = _u16(x).reshape(sp.rows, sp.cols)
        rc, rs, _ = oracle.quantize(xh, sp.fmt, PT)
        assert _u32(scales)[0] == rs.view(np.uint32)[0], sp.name
        assert np.array_equal(codes.cpu().numpy(), rc), sp.name
        rd = oracle.dequantize(rc, sp.fmt, PT, rs)
        assert np.array_equal(_u32(deq), rd.reshape(-1).view(np.uint32)), sp.name


def test_special_values_4gib_all_modes(dev):
    rng = np.random.default_rng(55)
    blocks_checked = elems_checked = 0
    for sp in synth.special_values_4gib():
        x = sp.full(dev)
        n = sp.rows * sp.cols
        xf = x.float()
        finite = torch.isfinite(xf)
        expect_nf = int((~finite).any().item())
        amax = torch.where(finite, xf.abs(), torch.zeros_like(xf)).max().item()
        del xf, finite
        samp = np.unique(np.concatenate([rng.integers(0, n, 200000), np.arange(256),
                                         np.arange(n - 256, n)]))
        ts = torch.from_numpy(samp)
        xs = sp.gen(ts).numpy().astype(np.uint16)
        xs_f32 = (xs.astype(np.uint32) << 16).view(np.float32)
        for fmt in (gs.FP8_E4M3, gs.FP8_E5M2):
            for gran in (PT, B1, B128):
                for mode in (gs.FP8_SCALE_FROM_AMAX, gs.FP8_SCALE_GIVEN):
                    nf = torch.zeros(1, dtype=torch.int32, device=dev)
                    sc = None
                    if mode == gs.FP8_SCALE_GIVEN:
                        sc = torch.ones(gs.scale_shape(sp.rows, sp.cols, gran),
                                        dtype=torch.float32, device=dev)
                    codes, scales = gs.fp8_quantize(x, fmt, gran, mode, scales=sc, nonfinite=nf)
                    deq = gs.fp8_dequantize(codes, fmt, gran, scales)
                    torch.cuda.synchronize()
                    assert int(nf.item()) == expect_nf
                    tag = (sp.name, fmt, gran, mode)
                    if mode == gs.FP8_SCALE_GIVEN:
                        ref = oracle.cast(xs_f32, 1.0, fmt)
                        got = codes.view(-1)[ts.to(dev)].cpu().numpy()
                        assert np.array_equal(got, ref), tag
                        rd = oracle.dequantize(ref.reshape(1, -1), fmt, PT, np.float32([1.0]))
                        assert np.array_equal(_u32(deq.view(-1)[ts.to(dev)]),
                                              rd.reshape(-1).view(np.uint32)), tag
                        elems_checked += got.size
                    elif gran == PT:
                        s_ref = oracle.scale_from_amax(amax, fmt)
                        assert _u32(scales)[0] == np.float32(s_ref).view(np.uint32), tag
                        ref = oracle.cast(xs_f32, float(s_ref), fmt)
                        got = codes.view(-1)[ts.to(dev)].cpu().numpy()
                        assert np.array_equal(got, ref), tag
                        elems_checked += got.size
                    else:
                        blocks_checked += _check_blocks(sp, codes, scales, deq, gran, fmt, rng,
                                                        400 if gran == B1 else 6)
                    del codes, scales, deq
        del x
        torch.cuda.empty_cache()
    print("special values: %d blocks and %d sampled elements checked" % (blocks_checked, elems_checked))
    assert blocks_checked >= 4 * 2 * (380 + 6) and elems_checked >= 4 * 2 * 4 * 190000


def _check_row32_blocks(x_spec, codes, scales, deq, mx, fmt, rng, nsample):
    """Sampled 1x32 blocks (FP32 scales, or MX E8M0 bytes when mx) against
    the oracle on the block regenerated on the host."""
    rows, cols = x_spec.rows, x_spec.cols
    nb = rows * (cols // 32)
    blocks = np.unique(np.concatenate([rng.integers(0, nb, nsample), [0, nb - 1]]))
    for b in blocks:
        r, j = divmod(int(b), cols // 32)
        idx = torch.arange(r * cols + j * 32, r * cols + j * 32 + 32)
        xb = x_spec.gen(idx).numpy().astype(np.uint16).reshape(1, 32)
        sl = (slice(r, r + 1), slice(j * 32, (j + 1) * 32))
        if mx:
            rc, rs, _ = oracle.quantize_mx(xb, fmt)
            rd = oracle.dequantize_mx(rc, fmt, rs)
            assert int(scales[r, j].item()) == int(rs[0, 0]), b
        else:
            rc, rs, _ = oracle.quantize(xb, fmt, PT)
            rd = oracle.dequantize(rc, fmt, PT, rs)
            assert _u32(scales[r, j:j + 1])[0] == rs.view(np.uint32)[0], b
        assert np.array_equal(codes[sl].cpu().numpy(), rc), b
        assert np.array_equal(_u32(deq[sl]).reshape(-1), rd.reshape(-1).view(np.uint32)), b
    return len(blocks)


def test_row32_and_mx_blocks_at_full_size(dev):
    """1x32 (FP32 scales) and MX 1x32 (E8M0) on the DeepSeek-V3 activation
    shape and on the four 16384x32768 special-value tensors: sampled blocks
    against the oracle, and the nonfinite flag over the whole tensor."""
    rng = np.random.default_rng(66)
    act = synth.deepseek_v3_blocks()[0]
    checked = 0
    for sp, fmts, nsample in [(act, (gs.FP8_E4M3,), 3000)] + \
            [(s, (gs.FP8_E4M3, gs.FP8_E5M2), 400) for s in synth.special_values_4gib()]:
        x = sp.full(dev)
        expect_nf = None
        for fmt in fmts:
            for mx in (False, True):
                nf = torch.zeros(1, dtype=torch.int32, device=dev)
                if mx:
                    codes, scales = gs.fp8_quantize_mx(x, fmt, nonfinite=nf)
                    deq = gs.fp8_dequantize_mx(codes, fmt, scales)
                else:
                    codes, scales = gs.fp8_quantize(x, fmt, gs.FP8_BLOCK_1x32, nonfinite=nf)
                    deq = gs.fp8_dequantize(codes, fmt, gs.FP8_BLOCK_1x32, scales)
                torch.cuda.synchronize()
                if expect_nf is None:
                    expect_nf = int((~torch.isfinite(x.float())).any().item())
                assert int(nf.item()) == expect_nf, (sp.name, fmt, mx)
                checked += _check_row32_blocks(sp, codes, scales, deq, mx, fmt, rng, nsample)
                del codes, scales, deq
        del x
        torch.cuda.empty_cache()
    assert checked >= 2 * 2900 + 4 * 2 * 2 * 380


def test_tensors_above_2_32_elements(dev):
    """Maximum sizes: one FP16 gradient tensor of 2^32 + 6149 elements and
    one 32896x131072 BF16 matrix (4.31e9 elements; the 1x128 and dequantize
    grids are capped and stride).  Sampled outputs around the 2^31 and 2^32
    element boundaries and at both ends against the oracle; an Inf past
    2^32 sets the flag; the exact sum of squares against an FP64 sum."""
    n = (1 << 32) + 3 * 2048 + 5
    g = synth.GradSet(seed=7007, scale=2.0 ** 15, log2_lo=-18.0, log2_hi=12.0, steps=1)
    g.tensors = [synth.GradSpec("big", n, 1)]
    grad = g.full(0, dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    S = torch.tensor([g.scale], dtype=torch.float32, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.zeros(2, dtype=torch.int64, device=dev)
    nsq = torch.zeros(1, dtype=torch.float64, device=dev)
    gs.gs_unscale_check_sumsq([grad], [out], S, f, acc, nsq)
    torch.cuda.synchronize()
    assert int(f.item()) == 0
    rng = np.random.default_rng(77)
    edges = [np.arange(0, 4096), np.arange(n - 4096, n),
             np.arange((1 << 31) - 2048, (1 << 31) + 2048), np.arange((1 << 32) - 2048, (1 << 32) + 2048)]
    idx = np.unique(np.concatenate(edges + [rng.integers(0, n, 50000)]))
    ti = torch.from_numpy(idx)
    bits = g.gen(0, ti).numpy().astype(np.uint16)
    ref, _ = oracle.unscale_check([bits], g.scale)
    assert np.array_equal(_u32(out[ti.to(dev)]), ref[0].view(np.uint32))
    tot = 0.0
    for lo in range(0, n, 1 << 28):
        tot += float((out[lo:lo + (1 << 28)].double() ** 2).sum().item())
    assert abs(float(nsq.item()) - tot) <= 1e-12 * tot
    pos = (1 << 32) + 7
    grad[pos:pos + 1].fill_(float("inf"))
    gs.gs_unscale_check([grad], [out], S, f)
    torch.cuda.synchronize()
    assert int(f.item()) == 1 and out[pos].item() == float("inf")
    del grad, out
    torch.cuda.empty_cache()

    sp = synth.BitsSpec("big_random", 32896, 131072, 7007, 2, "random")
    x = sp.full(dev)
    for gran in (B1, B128):
        codes, scales = gs.fp8_quantize(x, gs.FP8_E4M3, gran)
        deq = gs.fp8_dequantize(codes, gs.FP8_E4M3, gran, scales)
        torch.cuda.synchronize()
        nb = _check_blocks(sp, codes, scales, deq, gran, gs.FP8_E4M3, rng, 600 if gran == B1 else 20)
        assert nb >= (500 if gran == B1 else 15)
        # the first and last block of the row that starts at element 2^32
        if gran == B1:
            r = (1 << 32) // sp.cols
            for j in (0, sp.cols // 128 - 1):
                idx = torch.arange(r * sp.cols + j * 128, r * sp.cols + j * 128 + 128)
                xb = sp.gen(idx).numpy().astype(np.uint16).reshape(1, 128)
                rc, rs, _ = oracle.quantize(xb, gs.FP8_E4M3, PT)
                assert np.array_equal(codes[r, j * 128:(j + 1) * 128].cpu().numpy(), rc.reshape(-1))
        del codes, scales, deq
    codes, sc = gs.fp8_quantize_mx(x, gs.FP8_E5M2)
    deq = gs.fp8_dequantize_mx(codes, gs.FP8_E5M2, sc)
    torch.cuda.synchronize()
    assert _check_row32_blocks(sp, codes, sc, deq, True, gs.FP8_E5M2, rng, 600) >= 500
