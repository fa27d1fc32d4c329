"""GPU parity: unscale + exact gradient sum of squares (gs_unscale_check_sumsq)
through the C ABI against the oracle: the outputs and flag bit for bit, the
128-bit running total exactly, norm_sq bit for bit.  At the full Llama-3-8B
gradient size, properties that hold at any size: the total does not depend on
how the list is split into calls, an injected Inf removes exactly that
element's square, and the norm agrees with an independent FP64 sum."""
import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu

M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _to_dev(h: np.ndarray, dev):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.float16).to(dev)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def _acc(dev, start=(0, 0)):
    lo, hi = start
    return torch.tensor([lo if lo < (1 << 63) else lo - (1 << 64),
                         hi if hi < (1 << 63) else hi - (1 << 64)], dtype=torch.int64, device=dev)


def _acc_value(t):
    lo, hi = (int(v) & M64 for v in t.cpu().tolist())
    return lo, hi


def _f64_bits(x) -> int:
    return int(np.float64(x).view(np.uint64))


def _run(grads, outs, S, dev, start=(0, 0)):
    Sd = torch.tensor([S], dtype=torch.float32, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = _acc(dev, start)
    ns = torch.zeros(1, dtype=torch.float64, device=dev)
    gs.gs_unscale_check_sumsq(grads, outs, Sd, f, acc, ns)
    torch.cuda.synchronize()
    return int(f.item()), _acc_value(acc), float(ns.item())


def _check(host, grads, outs, S, dev, start=(0, 0), tag=""):
    flag, acc, ns = _run(grads, outs, S, dev, start)
    ref, rflag, racc, rns = oracle.unscale_check_sumsq(host, S, sumsq=start)
    for o, r in zip(outs, ref):
        assert np.array_equal(_bits(o), r.view(np.uint32)), tag
    assert flag == rflag, tag
    assert acc == tuple(racc), (tag, acc, racc)
    assert _f64_bits(ns) == _f64_bits(rns), (tag, ns, rns)
    return acc


SCALES = [2.0 ** k for k in range(-20, 41, 5)] + [3.0, 1000.0, 1e-30, 7e-39, 3.0e38,
                                                  float("inf")]


def test_every_fp16_pattern(dev):
    """All 65536 FP16 patterns in one tensor (Inf and NaN included, so the
    recompute of a lane's share runs), and the same patterns as 8 tensors."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = _to_dev(h, dev)
    o = torch.empty(65536, dtype=torch.float32, device=dev)
    for S in SCALES:
        _check([h], [g], [o], S, dev, tag=S)
    parts = np.split(h, 8)
    gp = [_to_dev(p, dev) for p in parts]
    op = [torch.empty(p.size, dtype=torch.float32, device=dev) for p in parts]
    _check(parts, gp, op, 65536.0, dev, tag="split")


def test_tiny_gradset_50_steps(dev):
    g = synth.tiny_gradset()
    host = [synth.as_u16_numpy(synth.to_f16_tensor(g.gen(t, torch.arange(sp.numel))))
            for t, sp in enumerate(g.tensors)]
    grads = [_to_dev(x, dev) for x in host]
    outs = [torch.empty(x.size, dtype=torch.float32, device=dev) for x in host]
    S = torch.tensor([g.scale], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    acc = torch.zeros(2, dtype=torch.int64, device=dev)
    ns = torch.zeros(1, dtype=torch.float64, device=dev)
    R = oracle.ScalerState(g.scale)
    for step in range(1, g.steps + 1):
        saved = []
        for (t, i, bits) in g.injections.get(step, []):
            saved.append((t, i, host[t][i]))
            host[t][i] = bits
            grads[t][i:i + 1] = _to_dev(np.array([bits], np.uint16), dev)
        acc.zero_()
        gs.gs_unscale_check_sumsq(grads, outs, S, found, acc, ns)
        ref, rflag, racc, rns = oracle.unscale_check_sumsq(host, float(R.S))
        torch.cuda.synchronize()
        for t, (o, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(_bits(o), r.view(np.uint32)), (step, t)
        assert int(found.item()) == rflag, step
        assert _acc_value(acc) == tuple(racc), step
        assert _f64_bits(ns.item()) == _f64_bits(rns), step
        R.found_inf.value = rflag
        gs.gs_update_scale(S, tracker, found, 2.0, 0.5, 2000)
        oracle.update_scale(R, 2.0, 0.5, 2000)
        for (t, i, old) in saved:
            host[t][i] = old
            grads[t][i:i + 1] = _to_dev(np.array([old], np.uint16), dev)
    torch.cuda.synchronize()
    assert float(S.item()) == float(R.S) == 8192.0


def test_ragged_misaligned_nonfinite_and_empty(dev):
    """Sizes around the 2048-element chunk and the 8-element vector, bases
    offset by 0..7 elements (the element-wise path), Inf/NaN scattered over
    both paths, empty tensors in the list."""
    rng = np.random.default_rng(19)
    sizes = [0, 1, 7, 8, 9, 2047, 2048, 2049, 3 * 2048 + 5, 0, 100000, 65536]
    host, grads, outs = [], [], []
    pool = torch.empty(1 << 20, dtype=torch.float16, device=dev)
    opool = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    off = 0
    for k, n in enumerate(sizes):
        h = rng.integers(0, 0x7C00, size=n, dtype=np.uint32).astype(np.uint16)
        h |= (rng.integers(0, 2, size=n).astype(np.uint16) << 15)
        if n > 100:
            pos = rng.choice(n, size=6, replace=False)
            h[pos] = [0x7C00, 0xFC00, 0x7E00, 0xFE01, 0x7C01, 0x7FFF]
        shift = 0 if k >= 10 else k % 8
        host.append(h)
        g = pool[off + shift: off + shift + n]
        if n:
            g.copy_(_to_dev(h, dev))
        o = opool[off + (0 if k >= 10 else 7 - shift): off + (0 if k >= 10 else 7 - shift) + n]
        grads.append(g)
        outs.append(o)
        off += n + 16
        off = (off + 7) // 8 * 8
    for S in (1024.0, 3.0, 2.0 ** -12):
        _check(host, grads, outs, S, dev, tag=S)


def test_running_total_carry_and_rounding(dev):
    """The running total: carry from the low into the high word, the RNE
    conversion of a total needing rounding and of an exact tie, and calls that
    accumulate (one list in pieces equals the list at once)."""
    rng = np.random.default_rng(5)
    h = rng.integers(0, 0x7C00, size=50000, dtype=np.uint32).astype(np.uint16)
    g = _to_dev(h, dev)
    o = torch.empty(h.size, dtype=torch.float32, device=dev)
    for start in [(M64, 5), (M64 - 12345, 0), ((1 << 60) + (1 << 7) + 1, 0),
                  ((1 << 60) + (1 << 7), 0), (3, 1 << 40), (0, (1 << 63) - 1)]:
        _check([h], [g], [o], 65536.0, dev, start=start, tag=start)
    # empty list: only the final step runs (adds nothing, writes the norm)
    for start in [((1 << 60) + (1 << 7) + 1, 0), ((1 << 60) + (1 << 7), 0), (M64, M64 >> 1)]:
        flag, acc, ns = _run([], [], 2.0, dev, start)
        _, rflag, racc, rns = oracle.unscale_check_sumsq([], 2.0, sumsq=start)
        assert acc == tuple(racc) == start and _f64_bits(ns) == _f64_bits(rns) and flag == 0
    # pieces: three calls adding into one total
    acc = _acc(dev)
    Sd = torch.tensor([4.0], dtype=torch.float32, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    ns = torch.zeros(1, dtype=torch.float64, device=dev)
    for a, b in ((0, 777), (777, 30001), (30001, 50000)):
        gs.gs_unscale_check_sumsq([g[a:b]], [o[a:b]], Sd, f, acc, ns)
    torch.cuda.synchronize()
    _, _, racc, rns = oracle.unscale_check_sumsq([h], 4.0)
    assert _acc_value(acc) == tuple(racc) and _f64_bits(ns.item()) == _f64_bits(rns)


def test_largest_magnitudes(dev):
    """Every element +-65504 (the largest chunk partials, X above 2^100) and
    the smallest subnormals."""
    n = 1 << 20
    big = np.where(np.arange(n) % 3 == 0, 0xFBFF, 0x7BFF).astype(np.uint16)
    small = np.where(np.arange(n) % 2 == 0, 0x0001, 0x8001).astype(np.uint16)
    gb, gsm = _to_dev(big, dev), _to_dev(small, dev)
    ob = torch.empty(n, dtype=torch.float32, device=dev)
    osm = torch.empty(n, dtype=torch.float32, device=dev)
    acc = _check([big, small], [gb, gsm], [ob, osm], 1.0, dev, tag="extremes")
    X = (acc[1] << 64) | acc[0]
    assert X == n * (65504 << 24) ** 2 + n


def test_llama3_8b_full_size_properties(dev):
    """291 tensors, 8,030,261,248 elements, in the benchmark's launch
    configuration.  (1) The exact total equals the sum of the totals of
    each tensor on its own (per-tensor calls accumulating); (2) with one
    +Inf injected, the total drops by exactly that element's square (checked
    against the oracle's value for it) and the flag is set; (3) norm_sq
    agrees with torch's FP64 sum of y^2 to 1e-12; (4) sampled outputs are
    the oracle's."""
    g = synth.llama3_8b_gradset()
    grads = [g.full(t, dev) for t in range(len(g.tensors))]
    outs = [torch.empty(sp.numel, dtype=torch.float32, device=dev) for sp in g.tensors]
    S = torch.tensor([g.scale], dtype=torch.float32, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(gs.gs_unscale_check_sumsq_workspace_size([sp.numel for sp in g.tensors]),
                     dtype=torch.uint8, device=dev)
    acc = _acc(dev)
    ns = torch.zeros(1, dtype=torch.float64, device=dev)
    gs.gs_unscale_check_sumsq(grads, outs, S, f, acc, ns, workspace=ws)
    torch.cuda.synchronize()
    whole = _acc_value(acc)
    assert int(f.item()) == 0
    X = (whole[1] << 64) | whole[0]
    # (3) independent FP64 sum of the outputs' squares, tensor by tensor
    ref = 0.0
    for o in outs:
        ref += float(torch.sum(o.double() ** 2).item())
    assert abs(float(ns.item()) - ref) <= 1e-12 * ref
    inv = float(np.float32(1.0) / np.float32(g.scale))
    assert float(ns.item()) == (float(X) * 2.0 ** -48) * (inv * inv)
    # (4) sampled outputs
    rng = np.random.default_rng(71)
    for t in rng.choice(len(g.tensors), size=24, replace=False):
        n = g.tensors[t].numel
        idx = np.unique(np.concatenate([rng.integers(0, n, 2048), [0, n - 1]]))
        ti = torch.from_numpy(idx)
        bits = g.gen(int(t), ti).numpy().astype(np.uint16)
        r, _ = oracle.unscale_check([bits], g.scale)
        assert np.array_equal(_bits(outs[int(t)][ti.to(dev)]), r[0].view(np.uint32)), t
    # (1) per-tensor calls into one total
    acc.zero_()
    for t in range(len(g.tensors)):
        gs.gs_unscale_check_sumsq([grads[t]], [outs[t]], S, f, acc, ns)
    torch.cuda.synchronize()
    assert _acc_value(acc) == whole
    # (2) one +Inf
    inj_t, inj_i, inj_bits = g.injections[2][0]
    orig = int(g.gen(inj_t, torch.tensor([inj_i]))[0]) & 0xFFFF
    _, _, one, _ = oracle.unscale_check_sumsq([np.array([orig], np.uint16)], g.scale)
    grads[inj_t][inj_i:inj_i + 1].fill_(float("inf"))
    acc.zero_()
    gs.gs_unscale_check_sumsq(grads, outs, S, f, acc, ns, workspace=ws)
    torch.cuda.synchronize()
    got = _acc_value(acc)
    assert int(f.item()) == 1
    assert ((got[1] << 64) | got[0]) == X - ((one[1] << 64) | one[0])
