"""CPU checks of the C ABI library: it loads, exports every function that
include/gs.h declares, and rejects bad arguments on the host (returning the
documented status before anything touches the GPU)."""
import ctypes
import os
import re

import pytest

import loss_scaling_fp8_amd as gs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                                r"([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_api():
    assert set(_declared_functions()) == set(gs.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gs.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code, name in ((0, "GS_OK"), (-1, "GS_ERR_NULL"), (-3, "GS_ERR_SHAPE"),
                       (-7, "GS_ERR_WORKSPACE"), (-8, "GS_ERR_HIP")):
        assert gs.status_string(code).startswith(name)
    assert "unknown" in gs.status_string(12345)


def test_workspace_size():
    assert gs.fp8_quantize_workspace_size(8192, 8192, gs.FP8_PER_TENSOR) == 32768
    assert gs.fp8_quantize_workspace_size(8192, 8192, gs.FP8_BLOCK_1x128) == 0
    assert gs.fp8_quantize_workspace_size(8192, 8192, gs.FP8_BLOCK_128x128) == 0


# Argument errors are found before any HIP call, so they are testable here.
FAKE = 1 << 40          # an aligned, never-dereferenced "device" address


def test_unscale_argument_errors():
    L = gs.lib()
    one = (ctypes.c_void_p * 1)(FAKE)
    n5 = (ctypes.c_int64 * 1)(5)
    assert L.gs_unscale_check(-1, one, one, n5, gs.GS_F16, FAKE, FAKE, None) == -2
    assert L.gs_unscale_check(1, one, one, n5, gs.GS_BF16, FAKE, FAKE, None) == -4
    assert L.gs_unscale_check(1, one, one, n5, gs.GS_F16, None, FAKE, None) == -1
    assert L.gs_unscale_check(1, one, one, n5, gs.GS_F16, FAKE, None, None) == -1
    assert L.gs_unscale_check(1, None, one, n5, gs.GS_F16, FAKE, FAKE, None) == -1
    nul = (ctypes.c_void_p * 1)(None)
    assert L.gs_unscale_check(1, nul, one, n5, gs.GS_F16, FAKE, FAKE, None) == -1
    neg = (ctypes.c_int64 * 1)(-3)
    assert L.gs_unscale_check(1, one, one, neg, gs.GS_F16, FAKE, FAKE, None) == -2
    odd = (ctypes.c_void_p * 1)(FAKE + 1)
    assert L.gs_unscale_check(1, odd, one, n5, gs.GS_F16, FAKE, FAKE, None) == -6
    assert L.gs_unscale_check(1, one, odd, n5, gs.GS_F16, FAKE, FAKE, None) == -6
    # nothing to do: returns OK without launching
    assert L.gs_unscale_check(0, None, None, None, gs.GS_F16, FAKE, FAKE, None) == 0
    zero = (ctypes.c_int64 * 1)(0)
    assert L.gs_unscale_check(1, nul, nul, zero, gs.GS_F16, FAKE, FAKE, None) == 0


def test_update_argument_errors():
    L = gs.lib()
    assert L.gs_update_scale(None, FAKE, FAKE, 2.0, 0.5, 2000, None, None) == -1
    assert L.gs_update_scale(FAKE, FAKE, FAKE, 2.0, 0.5, 0, None, None) == -5
    assert L.gs_update_scale(FAKE, FAKE, FAKE, float("inf"), 0.5, 10, None, None) == -5
    assert L.gs_update_scale(FAKE, FAKE, FAKE, 2.0, -0.5, 10, None, None) == -5
    assert L.gs_update_scale(FAKE, FAKE, FAKE, 2.0, 0.0, 10, None, None) == -5
    assert L.gs_update_scale(FAKE + 2, FAKE, FAKE, 2.0, 0.5, 10, None, None) == -6
    assert L.gs_update_scale(FAKE, FAKE, FAKE, 2.0, 0.5, 10, FAKE + 4, None) == -6


@pytest.mark.parametrize("args,code", [
    ((FAKE, 1, 128, 128, 0, 1, 0), -4),        # FP16 input not supported
    ((FAKE, 2, 128, 128, 2, 1, 0), -5),        # bad format
    ((FAKE, 2, 128, 128, 0, 4, 0), -5),        # bad granularity
    ((FAKE, 2, 128, 128, 0, 1, 2), -5),        # bad mode
    ((FAKE, 2, 128, 100, 0, 1, 0), -3),        # 1x128 needs cols % 128
    ((FAKE, 2, 100, 128, 0, 2, 0), -3),        # 128x128 needs rows % 128
    ((FAKE, 2, -1, 128, 0, 0, 0), -2),
    ((FAKE, 2, 1 << 32, 2, 0, 0, 0), -2),
    ((None, 2, 128, 128, 0, 1, 0), -1),
    ((FAKE + 2, 2, 128, 128, 0, 1, 0), -6),
])
def test_quantize_argument_errors(args, code):
    L = gs.lib()
    x, dt, r, c, fmt, gran, mode = args
    assert L.fp8_quantize(x, dt, r, c, fmt, gran, mode, FAKE, FAKE, None, None, 0, None) == code


def test_quantize_workspace_and_output_errors():
    L = gs.lib()
    # per-tensor amax mode without workspace
    assert L.fp8_quantize(FAKE, 2, 64, 64, 0, 0, 0, FAKE, FAKE, None, None, 0, None) == -7
    assert L.fp8_quantize(FAKE, 2, 64, 64, 0, 0, 0, FAKE, FAKE, None, FAKE, 16, None) == -7
    assert L.fp8_quantize(FAKE, 2, 64, 64, 0, 0, 0, None, FAKE, None, FAKE, 32768, None) == -1
    assert L.fp8_quantize(FAKE, 2, 64, 64, 0, 0, 0, FAKE, None, None, FAKE, 4096, None) == -1


def test_dequantize_argument_errors():
    L = gs.lib()
    assert L.fp8_dequantize(FAKE, 128, 100, 0, 1, FAKE, FAKE, None) == -3
    assert L.fp8_dequantize(FAKE, 128, 128, 5, 1, FAKE, FAKE, None) == -5
    assert L.fp8_dequantize(None, 128, 128, 0, 1, FAKE, FAKE, None) == -1
    assert L.fp8_dequantize(FAKE, 128, 128, 0, 1, FAKE, FAKE + 8, None) == -6
    assert L.fp8_dequantize(None, 0, 128, 0, 1, None, None, None) == 0   # empty: nothing to do


def test_quantize_delayed_argument_errors():
    L = gs.lib()
    f = L.fp8_quantize_delayed
    args = dict(x=FAKE, dt=2, r=64, c=64, fmt=0, st=FAKE, hist=FAKE, hl=16, pos=FAKE,
                codes=FAKE, used=FAKE, nf=None, ws=FAKE, wsb=32768)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["dt"], a["r"], a["c"], a["fmt"], a["st"], a["hist"], a["hl"],
                 a["pos"], a["codes"], a["used"], a["nf"], a["ws"], a["wsb"], None)
    assert call(dt=1) == -4
    assert call(fmt=3) == -5
    assert call(hl=0) == -5
    assert call(hl=1025) == -5
    assert call(r=-1) == -2
    assert call(x=None) == -1
    assert call(st=None) == -1
    assert call(hist=None) == -1
    assert call(pos=None) == -1
    assert call(used=None) == -1
    assert call(x=FAKE + 8) == -6
    assert call(pos=FAKE + 2) == -6
    assert call(ws=None) == -7
    assert call(wsb=100) == -7


def test_unscale_sumsq_workspace_size():
    assert gs.gs_unscale_check_sumsq_workspace_size([]) == 16 * 1024
    assert gs.gs_unscale_check_sumsq_workspace_size([1, 2048, 2049, 0]) == 16 * (1 + 1 + 2 + 1024)
    assert gs.gs_unscale_check_sumsq_workspace_size([-1]) == 0


def test_unscale_sumsq_argument_errors():
    L = gs.lib()
    f = L.gs_unscale_check_sumsq
    one = (ctypes.c_void_p * 1)(FAKE)
    n5 = (ctypes.c_int64 * 1)(5)
    ws = 16 * 1025
    args = dict(n=1, g=one, o=one, nums=n5, dt=gs.GS_F16, s=FAKE, fi=FAKE, sq=FAKE, ns=FAKE,
                ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["n"], a["g"], a["o"], a["nums"], a["dt"], a["s"], a["fi"], a["sq"], a["ns"],
                 a["ws"], a["wsb"], None)
    assert call(n=-1) == -2
    assert call(dt=gs.GS_BF16) == -4
    for k in ("s", "fi", "sq", "ns", "g", "o", "nums"):
        assert call(**{k: None}) == -1, k
    assert call(nums=(ctypes.c_int64 * 1)(-3)) == -2
    assert call(sq=FAKE + 4) == -6
    assert call(ns=FAKE + 4) == -6
    assert call(g=(ctypes.c_void_p * 1)(FAKE + 1)) == -6
    assert call(ws=None) == -7
    assert call(wsb=ws - 1) == -7
    assert call(ws=FAKE + 8) == -6


def test_update_hysteresis_argument_errors():
    L = gs.lib()
    f = L.gs_update_scale_hysteresis
    args = dict(s=FAKE, t=FAKE, h=FAKE, fi=FAKE, g=2.0, b=0.5, w=1000, H=2, c=0, m=1.0, k=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["s"], a["t"], a["h"], a["fi"], a["g"], a["b"], a["w"], a["H"], a["c"], a["m"],
                 a["k"], None)
    for k in ("s", "t", "h", "fi"):
        assert call(**{k: None}) == -1, k
    assert call(h=FAKE + 2) == -6
    assert call(k=FAKE + 4) == -6
    assert call(w=0) == -5
    assert call(H=0) == -5
    assert call(c=2) == -5
    assert call(m=-1.0) == -5
    assert call(m=float("nan")) == -5
    assert call(g=float("inf")) == -5
    assert call(b=0.0) == -5


def test_mx_and_1x32_argument_errors():
    L = gs.lib()
    q, d = L.fp8_quantize_mx, L.fp8_dequantize_mx
    assert q(FAKE, 1, 4, 64, 0, FAKE, FAKE, None, None) == -4          # FP16 input
    assert q(FAKE, 2, 4, 64, 2, FAKE, FAKE, None, None) == -5          # bad format
    assert q(FAKE, 2, 4, 48, 0, FAKE, FAKE, None, None) == -3          # cols % 32
    assert q(FAKE, 2, -1, 64, 0, FAKE, FAKE, None, None) == -2
    assert q(None, 2, 4, 64, 0, FAKE, FAKE, None, None) == -1
    assert q(FAKE, 2, 4, 64, 0, FAKE, None, None, None) == -1
    assert q(FAKE + 8, 2, 4, 64, 0, FAKE, FAKE, None, None) == -6
    assert q(None, 2, 0, 64, 0, None, None, None, None) == 0          # empty
    assert d(FAKE, 4, 48, 0, FAKE, FAKE, None) == -3
    assert d(FAKE, 4, 64, 0, None, FAKE, None) == -1
    assert d(FAKE, 4, 64, 0, FAKE, FAKE + 4, None) == -6
    assert d(None, 0, 64, 0, None, None, None) == 0
    assert L.fp8_quantize(FAKE, 2, 4, 48, 0, 3, 0, FAKE, FAKE, None, None, 0, None) == -3
    assert L.fp8_dequantize(FAKE, 4, 48, 0, 3, FAKE, FAKE, None) == -3
    assert L.fp8_quantize(FAKE, 2, 4, 64, 0, 4, 0, FAKE, FAKE, None, None, 0, None) == -5


def _descriptor_layout(ins, outs, numels):
    """The documented chunk-descriptor layout of gs_unscale_list_descriptors."""
    d = []
    for a, b, n in zip(ins, outs, numels):
        if n == 0:
            continue
        scalar = 1 if (a | b) & 15 else 0
        for st in range(0, n, 2048):
            left = n - st
            ragged = left if left < 2048 else 0
            d.append(((a + 2 * st) | (ragged << 48), (b + 4 * st) | scalar))
    return d


def _call_descriptors(ins, outs, numels, capacity=None, with_out=True):
    L = gs.lib()
    n = len(numels)
    gi = (ctypes.c_void_p * max(n, 1))(*ins)
    go = (ctypes.c_void_p * max(n, 1))(*outs)
    nu = (ctypes.c_int64 * max(n, 1))(*numels)
    cap = capacity if capacity is not None else sum((x + 2047) // 2048 for x in numels)
    buf = (ctypes.c_uint64 * max(2 * cap, 2))()
    r = L.gs_unscale_list_descriptors(n, gi, go, nu, buf if with_out else None, cap)
    return r, [(buf[2 * k], buf[2 * k + 1]) for k in range(max(r, 0))] if with_out else None


def test_list_descriptors_layout():
    """The host-side chunking of the multi-tensor unscale: tensors in order,
    empty ones skipped, 2048-element chunks, the ragged count of each last
    chunk in bits 48-63, the element-wise flag for tensors whose input or
    output is not 16-byte aligned."""
    import random
    rnd = random.Random(5)
    sizes = [0, 1, 7, 2047, 2048, 2049, 4096, 6149, 0, 1_000_003, 65536, 3]
    # per-tensor bases 1 GiB apart, offset in 2-byte (input) and 4-byte
    # (output) steps: some tensors 16-byte aligned on both sides, some not
    ins = [(1 << 40) + (k << 30) + (0 if k % 2 == 0 else 2 * (k % 8)) for k in range(len(sizes))]
    outs = [(1 << 42) + (k << 31) + (0 if k % 2 == 0 else 4 * (1 + k % 3)) for k in range(len(sizes))]
    r, got = _call_descriptors(ins, outs, sizes)
    want = _descriptor_layout(ins, outs, sizes)
    assert r == len(want) == sum((n + 2047) // 2048 for n in sizes)
    assert got == want
    assert any(o & 1 for _, o in want) and any(not (o & 1) for _, o in want)
    # the count alone, and its agreement with the sum-of-squares workspace size
    r2, _ = _call_descriptors(ins, outs, sizes, with_out=False)
    assert r2 == r == gs.gs_unscale_check_sumsq_workspace_size(sizes) // 16 - 1024
    # random lists
    for trial in range(20):
        m = rnd.randint(1, 30)
        ns = [rnd.choice([0, rnd.randint(1, 5000), rnd.randint(1, 300000)]) for _ in range(m)]
        ii = [(1 << 40) + 2 * rnd.randint(0, 1 << 30) for _ in ns]
        oo = [(1 << 41) + 4 * rnd.randint(0, 1 << 30) for _ in ns]
        assert _call_descriptors(ii, oo, ns)[1] == _descriptor_layout(ii, oo, ns)


def test_list_descriptors_errors():
    # capacity smaller than the count
    r, _ = _call_descriptors([FAKE], [FAKE], [5000], capacity=2)
    assert r == -2
    # an address reaching 2^48
    r, _ = _call_descriptors([(1 << 48) - 64], [FAKE], [100])
    assert r == -5
    r, _ = _call_descriptors([FAKE], [(1 << 48) - 128], [100])
    assert r == -5
    # alignment to the element size, negative counts, empty list
    assert _call_descriptors([FAKE + 1], [FAKE], [10])[0] == -6
    assert _call_descriptors([FAKE], [FAKE + 2], [10])[0] == -6
    assert _call_descriptors([FAKE], [FAKE], [-1])[0] == -2
    assert _call_descriptors([], [], [])[0] == 0


def test_dequantize_bf16_argument_errors():
    L = gs.lib()
    assert L.fp8_dequantize_bf16(FAKE, 128, 100, 0, 1, FAKE, FAKE, None) == -3
    assert L.fp8_dequantize_bf16(FAKE, 128, 128, 5, 1, FAKE, FAKE, None) == -5
    assert L.fp8_dequantize_bf16(FAKE, 128, 128, 0, 4, FAKE, FAKE, None) == -5
    assert L.fp8_dequantize_bf16(None, 128, 128, 0, 1, FAKE, FAKE, None) == -1
    assert L.fp8_dequantize_bf16(FAKE, 128, 128, 0, 1, FAKE, FAKE + 8, None) == -6
    assert L.fp8_dequantize_bf16(FAKE, -1, 128, 0, 1, FAKE, FAKE, None) == -2
    assert L.fp8_dequantize_bf16(None, 0, 128, 0, 1, None, None, None) == 0   # empty: nothing to do
