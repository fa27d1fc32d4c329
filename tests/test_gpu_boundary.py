"""GPU checks of the boundary's own machinery, through the C ABI against the
oracle: the device cache of gradient-list descriptors under eviction, calls
from several host threads on their own streams, and whole steps captured in
HIP graphs (after the list's first call, the library allocates nothing and
records no memset) -- the core step, and one that calls every other entry
point -- replayed with eager work between the replays."""
import threading

import numpy as np
import pytest
import torch

import loss_scaling_fp8_amd as gs
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _to_dev(h, dev):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.float16).to(dev)


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _random_f16(rng, n):
    h = rng.integers(0, 0x7C00, size=n, dtype=np.uint32).astype(np.uint16)
    return h | (rng.integers(0, 2, size=n).astype(np.uint16) << 15)


def test_descriptor_cache_eviction(dev):
    """80 distinct lists (the cache keeps 64): every call, including the
    repeat of an evicted list, matches the oracle."""
    rng = np.random.default_rng(81)
    lists = []
    for k in range(80):
        sizes = [int(v) for v in rng.integers(1, 5000, size=3)]
        host = [_random_f16(rng, n) for n in sizes]
        lists.append((host, [_to_dev(h, dev) for h in host],
                      [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]))
    S = torch.tensor([256.0], dtype=torch.float32, device=dev)
    for rnd in range(2):                    # the second round repeats lists evicted in the first
        for k in (list(range(80)) if rnd == 0 else [0, 1, 2, 79, 40, 0]):
            host, g, o = lists[k]
            f = torch.zeros(1, dtype=torch.int32, device=dev)
            for out in o:
                out.fill_(-1.0)
            gs.gs_unscale_check(g, o, S, f)
            ref, rf = oracle.unscale_check(host, 256.0)
            torch.cuda.synchronize()
            for out, r in zip(o, ref):
                assert np.array_equal(_bits(out), r.view(np.uint32)), (rnd, k)
            assert int(f.item()) == rf


def test_concurrent_host_threads_on_own_streams(dev):
    """Four host threads, each with its own stream and gradient list, call
    the unscale and the quantizer 25 times; every result matches the oracle
    (the descriptor cache is shared and locked)."""
    rng = np.random.default_rng(82)
    work = []
    for t in range(4):
        host = [_random_f16(rng, n) for n in (3000 + t, 77, 20000)]
        xq = (rng.standard_normal((64, 256)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        work.append((host, xq))
    errors = []

    def run(t):
        try:
            host, xq = work[t]
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                g = [_to_dev(h, dev) for h in host]
                o = [torch.empty(h.size, dtype=torch.float32, device=dev) for h in host]
                x = torch.from_numpy(xq.view(np.int16)).view(torch.bfloat16).to(dev)
                S = torch.tensor([1024.0], dtype=torch.float32, device=dev)
                f = torch.zeros(1, dtype=torch.int32, device=dev)
                for _ in range(25):
                    gs.gs_unscale_check(g, o, S, f)
                    codes, scales = gs.fp8_quantize(x, gs.FP8_E4M3, gs.FP8_BLOCK_1x128)
                s.synchronize()
                ref, _ = oracle.unscale_check(host, 1024.0)
                for out, r in zip(o, ref):
                    assert np.array_equal(_bits(out), r.view(np.uint32))
                rc, rs, _ = oracle.quantize(xq, gs.FP8_E4M3, gs.FP8_BLOCK_1x128)
                assert np.array_equal(codes.cpu().numpy(), rc)
                assert np.array_equal(scales.cpu().numpy().reshape(-1).view(np.uint32), rs.view(np.uint32))
        except Exception as e:          # noqa: BLE001 -- reported below
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=run, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors


def test_step_captured_in_a_hip_graph(dev):
    """unscale + check, update, 1x128 quantize and dequantize captured once
    (the list is cached by an eager call first) and replayed 6 times; an Inf
    is written eagerly into the input before replay 3 and removed after it;
    every replay matches the oracle (outputs, flag consumed, S / tracker /
    skips, codes, scales, dequantized values)."""
    g = synth.tiny_gradset()
    host = [synth.as_u16_numpy(synth.to_f16_tensor(g.gen(t, torch.arange(sp.numel))))
            for t, sp in enumerate(g.tensors)]
    grads = [_to_dev(h, dev) for h in host]
    outs = [torch.empty(h.size, dtype=torch.float32, device=dev) for h in host]
    q = synth.QuantSpec("graph", 256, 512, 0, 1, 7, 7, "gauss", 1.0, 0.01, 300.0)
    bits = q.gen(torch.arange(256 * 512)).to(torch.int32).to(torch.int16)
    xh = bits.numpy().view(np.uint16).reshape(256, 512)
    x = bits.view(torch.bfloat16).reshape(256, 512).to(dev)
    codes = torch.empty((256, 512), dtype=torch.uint8, device=dev)
    scales = torch.empty(gs.scale_shape(256, 512, gs.FP8_BLOCK_1x128), dtype=torch.float32, device=dev)
    deq = torch.empty((256, 512), dtype=torch.float32, device=dev)
    S = torch.tensor([g.scale], dtype=torch.float32, device=dev)
    tracker = torch.zeros(1, dtype=torch.int32, device=dev)
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    skips = torch.zeros(1, dtype=torch.int64, device=dev)

    def step():
        gs.gs_unscale_check(grads, outs, S, found)
        gs.gs_update_scale(S, tracker, found, 2.0, 0.5, 4, skips)
        gs.fp8_quantize(x, gs.FP8_E4M3, gs.FP8_BLOCK_1x128, gs.FP8_SCALE_FROM_AMAX, codes, scales)
        gs.fp8_dequantize(codes, gs.FP8_E4M3, gs.FP8_BLOCK_1x128, scales, deq)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # caches the descriptors, warms up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    S.fill_(g.scale)
    tracker.zero_()
    found.zero_()
    skips.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    R = oracle.ScalerState(g.scale)
    rc, rs, _ = oracle.quantize(xh, gs.FP8_E4M3, gs.FP8_BLOCK_1x128)
    rd = oracle.dequantize(rc, gs.FP8_E4M3, gs.FP8_BLOCK_1x128, rs)
    inj_t, inj_i = 5, 17
    for r in range(1, 7):
        if r == 3:
            host[inj_t][inj_i] = 0x7C00
            grads[inj_t][inj_i:inj_i + 1] = _to_dev(np.array([0x7C00], np.uint16), dev)
        for o in outs:
            o.fill_(-2.0)                         # eager work between replays
        codes.zero_()
        deq.zero_()
        graph.replay()
        ref, rf = oracle.unscale_check(host, float(R.S))
        R.found_inf.value = rf
        oracle.update_scale(R, 2.0, 0.5, 4)
        torch.cuda.synchronize()
        for o, rr in zip(outs, ref):
            assert np.array_equal(_bits(o), rr.view(np.uint32)), r
        assert (float(S.item()), int(tracker.item()), int(skips.item()), int(found.item())) == \
            (float(R.S), R.tracker.value, R.skips.value, 0), r
        assert np.array_equal(codes.cpu().numpy(), rc), r
        assert np.array_equal(scales.cpu().numpy().reshape(-1).view(np.uint32), rs.view(np.uint32)), r
        assert np.array_equal(deq.cpu().numpy().view(np.uint32), rd.view(np.uint32)), r
        if r == 3:
            orig = int(g.gen(inj_t, torch.tensor([inj_i]))[0]) & 0xFFFF
            host[inj_t][inj_i] = orig
            grads[inj_t][inj_i:inj_i + 1] = _to_dev(np.array([orig], np.uint16), dev)
    # closed form: replays 1-2 clean, 3 skipped (S halves), 4-6 clean (tracker 3 < 4)
    assert (float(R.S), R.skips.value, R.tracker.value) == (g.scale / 2, 1, 3)


def _bf16_bits(x):
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_extended_step_captured_in_a_hip_graph(dev):
    """The other entry points captured once and replayed 6 times: unscale with
    the exact sum of squares, the hysteresis update (Infs before replays 3
    and 4 spend the budget, then lower S), a delayed-scaling step, a
    per-tensor E5M2 quantize with its BF16 dequantize, a 128x128 quantize
    with its BF16 dequantize, and an MX quantize + dequantize.  The input
    matrix is rewritten eagerly between replays (a new magnitude each time),
    so the delayed history moves; every replay matches the oracle."""
    rng = np.random.default_rng(77)
    sizes = (3000, 20000, 517)
    host = [_random_f16(rng, n) & np.uint16(0xBBFF) for n in sizes]   # finite, |g| < 1
    grads = [_to_dev(h, dev) for h in host]
    outs = [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]
    R, C = 256, 512
    xs = [_bf16_bits(rng.standard_normal((R, C)).astype(np.float32) * np.float32(2.0 ** (r % 3 - 1)))
          for r in range(7)]
    x = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    ws_sq = torch.empty(gs.gs_unscale_check_sumsq_workspace_size(list(sizes)), dtype=torch.uint8, device=dev)
    ws_pt = torch.empty(gs.fp8_quantize_workspace_size(R, C, gs.FP8_PER_TENSOR), dtype=torch.uint8, device=dev)
    ws_dl = torch.empty(gs.fp8_quantize_workspace_size(R, C, gs.FP8_PER_TENSOR), dtype=torch.uint8, device=dev)
    S = torch.empty(1, dtype=torch.float32, device=dev)
    tr = torch.empty(1, dtype=torch.int32, device=dev)
    h = torch.empty(1, dtype=torch.int32, device=dev)
    found = torch.empty(1, dtype=torch.int32, device=dev)
    skips = torch.empty(1, dtype=torch.int64, device=dev)
    acc = torch.empty(2, dtype=torch.int64, device=dev)
    nsq = torch.empty(1, dtype=torch.float64, device=dev)
    st = torch.empty(1, dtype=torch.float32, device=dev)
    hist = torch.empty(4, dtype=torch.float32, device=dev)
    pos = torch.empty(1, dtype=torch.int32, device=dev)
    c_dl = torch.empty((R, C), dtype=torch.uint8, device=dev)
    used = torch.empty(1, dtype=torch.float32, device=dev)
    c_pt = torch.empty((R, C), dtype=torch.uint8, device=dev)
    s_pt = torch.empty(1, dtype=torch.float32, device=dev)
    d_pt = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    c_tl = torch.empty((R, C), dtype=torch.uint8, device=dev)
    s_tl = torch.empty(gs.scale_shape(R, C, gs.FP8_BLOCK_128x128), dtype=torch.float32, device=dev)
    d_tl = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    c_mx = torch.empty((R, C), dtype=torch.uint8, device=dev)
    s_mx = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
    d_mx = torch.empty((R, C), dtype=torch.float32, device=dev)

    def reset():
        S.fill_(65536.0)
        tr.zero_()
        h.fill_(2)
        found.zero_()
        skips.zero_()
        st.fill_(1.0)
        hist.zero_()
        pos.zero_()

    def step():
        gs.gs_unscale_check_sumsq(grads, outs, S, found, acc, nsq, ws_sq)
        gs.gs_update_scale_hysteresis(S, tr, h, found, 2.0, 0.5, 3, 2, False, 1.0, skips)
        gs.fp8_quantize_delayed(x, gs.FP8_E4M3, st, hist, pos, c_dl, used, None, ws_dl)
        gs.fp8_quantize(x, gs.FP8_E5M2, gs.FP8_PER_TENSOR, gs.FP8_SCALE_FROM_AMAX, c_pt, s_pt, None, ws_pt)
        gs.fp8_dequantize_bf16(c_pt, gs.FP8_E5M2, gs.FP8_PER_TENSOR, s_pt, d_pt)
        gs.fp8_quantize(x, gs.FP8_E4M3, gs.FP8_BLOCK_128x128, gs.FP8_SCALE_FROM_AMAX, c_tl, s_tl)
        gs.fp8_dequantize_bf16(c_tl, gs.FP8_E4M3, gs.FP8_BLOCK_128x128, s_tl, d_tl)
        gs.fp8_quantize_mx(x, gs.FP8_E4M3, c_mx, s_mx)
        gs.fp8_dequantize_mx(c_mx, gs.FP8_E4M3, s_mx, d_mx)

    x.copy_(torch.from_numpy(xs[0].view(np.int16)).view(torch.bfloat16))
    reset()
    acc.zero_()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # caches the descriptors, warms up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    RS = oracle.HysteresisState(65536.0, 0, 2)
    RD = oracle.DelayedState(4, 1.0)
    inj_t, inj_i = 1, 4321
    for r in range(1, 7):
        bad = r in (3, 4)
        host[inj_t][inj_i] = 0x7C00 if bad else 0x3C00
        grads[inj_t][inj_i:inj_i + 1] = _to_dev(np.array([host[inj_t][inj_i]], np.uint16), dev)
        x.copy_(torch.from_numpy(xs[r].view(np.int16)).view(torch.bfloat16))
        acc.zero_()                              # the caller zeroes the running total per step
        for o in outs:
            o.fill_(-2.0)
        for t in (c_dl, c_pt, c_tl, c_mx, s_mx):
            t.zero_()
        for t in (d_pt, d_tl, d_mx):
            t.zero_()
        graph.replay()
        ref, rf, racc, rnsq = oracle.unscale_check_sumsq(host, float(RS.S))
        RS.found_inf.value = rf
        oracle.update_scale_hysteresis(RS, 2.0, 0.5, 3, 2, False, 1.0)
        rc_dl, ru, _ = oracle.quantize_delayed(xs[r], gs.FP8_E4M3, RD)
        rc_pt, rs_pt, _ = oracle.quantize(xs[r], gs.FP8_E5M2, gs.FP8_PER_TENSOR)
        rc_tl, rs_tl, _ = oracle.quantize(xs[r], gs.FP8_E4M3, gs.FP8_BLOCK_128x128)
        rc_mx, rs_mx, _ = oracle.quantize_mx(xs[r], gs.FP8_E4M3)
        torch.cuda.synchronize()
        for o, rr in zip(outs, ref):
            assert np.array_equal(_bits(o), rr.view(np.uint32)), r
        assert tuple(int(v) & ((1 << 64) - 1) for v in acc.cpu().tolist()) == tuple(racc), r
        assert float(nsq.item()) == rnsq, r
        assert (float(S.item()), int(tr.item()), int(h.item()), int(skips.item()), int(found.item())) == \
            (float(RS.S), RS.tracker.value, RS.h.value, RS.skips.value, 0), r
        assert np.array_equal(c_dl.cpu().numpy(), rc_dl), r
        assert np.float32(used.item()).view(np.uint32) == np.float32(ru).view(np.uint32), r
        assert np.array_equal(hist.cpu().numpy().view(np.uint32), RD.history.view(np.uint32)), r
        assert np.float32(st.item()).view(np.uint32) == RD.scale.view(np.uint32)[0], r
        assert np.array_equal(c_pt.cpu().numpy(), rc_pt), r
        assert np.array_equal(s_pt.cpu().numpy().view(np.uint32), rs_pt.reshape(-1).view(np.uint32)), r
        assert np.array_equal(d_pt.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.dequantize_bf16(rc_pt, gs.FP8_E5M2, gs.FP8_PER_TENSOR, rs_pt)), r
        assert np.array_equal(c_tl.cpu().numpy(), rc_tl), r
        assert np.array_equal(s_tl.cpu().numpy().reshape(-1).view(np.uint32), rs_tl.reshape(-1).view(np.uint32)), r
        assert np.array_equal(d_tl.view(torch.int16).cpu().numpy().view(np.uint16),
                              oracle.dequantize_bf16(rc_tl, gs.FP8_E4M3, gs.FP8_BLOCK_128x128, rs_tl)), r
        assert np.array_equal(c_mx.cpu().numpy(), rc_mx) and np.array_equal(s_mx.cpu().numpy(), rs_mx), r
        assert np.array_equal(_bits(d_mx), oracle.dequantize_mx(rc_mx, gs.FP8_E4M3, rs_mx).view(np.uint32)), r
    # closed form: replays 1-2 clean (tracker 2), 3 spends the budget, 4 lowers S, 5-6 clean
    assert (float(RS.S), RS.skips.value, RS.tracker.value) == (32768.0, 2, 2)


def _small_lists(rng, dev, count, seed_sizes=(2500, 301, 9000)):
    """`count` distinct gradient lists of similar sizes (so their descriptor
    buffers are interchangeable), as (host, device grads, device outputs)."""
    lists = []
    for k in range(count):
        sizes = [int(n + (k * 37) % 97) for n in seed_sizes]
        host = [_random_f16(rng, n) for n in sizes]
        lists.append((host, [_to_dev(h, dev) for h in host],
                      [torch.empty(n, dtype=torch.float32, device=dev) for n in sizes]))
    return lists


def test_list_captured_in_a_graph_survives_eviction(dev):
    """A list used while its stream captures a graph stays cached: after 80
    other lists have gone through the 64-list cache (evicting lists and
    reusing their retired descriptor buffers), replaying the graph still
    reads its own descriptors, and every replay and every eager call matches
    the oracle.  Every tensor stays alive to the end, so a wrong reuse could
    only misdirect writes into live buffers."""
    rng = np.random.default_rng(83)
    (host, g, o), = _small_lists(rng, dev, 1, (4000, 123, 30000))
    S = torch.tensor([512.0], dtype=torch.float32, device=dev)
    f = torch.zeros(1, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gs.gs_unscale_check(g, o, S, f)          # first call: builds and caches the list
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs.gs_unscale_check(g, o, S, f)
    torch.cuda.synchronize()
    others = _small_lists(rng, dev, 80)
    ref, rf = oracle.unscale_check(host, 512.0)
    for rnd in range(3):
        for k, (oh, og, oo) in enumerate(others):
            of = torch.zeros(1, dtype=torch.int32, device=dev)
            gs.gs_unscale_check(og, oo, S, of)
            if k % 9 == rnd:
                oref, orf = oracle.unscale_check(oh, 512.0)
                torch.cuda.synchronize()
                for out, r in zip(oo, oref):
                    assert np.array_equal(_bits(out), r.view(np.uint32)), (rnd, k)
                assert int(of.item()) == orf
        for out in o:
            out.fill_(-3.0)
        f.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for out, r in zip(o, ref):
            assert np.array_equal(_bits(out), r.view(np.uint32)), rnd
        assert int(f.item()) == rf


def test_evictions_while_another_thread_captures(dev):
    """Thread B pushes distinct gradient lists through the cache on its own
    stream (evictions, and retired descriptor buffers reused once the events
    of their last launches have completed) while thread A, on its own
    stream, repeatedly captures an unscale + update step in a HIP graph
    (thread-local capture mode, so that B may allocate and upload meanwhile)
    and replays each graph three times with eager work between the replays.
    Every result of both threads matches the oracle.  All tensors are made
    before the threads start and stay alive to the end."""
    rng = np.random.default_rng(84)
    (hA, gA, oA), = _small_lists(rng, dev, 1, (6000, 50, 20000))
    hA[1][7] = 0x7C00                           # an Inf: every replay overflows and skips
    gA[1][7:8] = _to_dev(np.array([0x7C00], np.uint16), dev)
    SA = torch.tensor([2.0 ** 20], dtype=torch.float32, device=dev)
    trA = torch.zeros(1, dtype=torch.int32, device=dev)
    fA = torch.zeros(1, dtype=torch.int32, device=dev)
    listsB = _small_lists(rng, dev, 160)
    SB = torch.tensor([128.0], dtype=torch.float32, device=dev)
    fB = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in listsB]
    torch.cuda.synchronize()
    errors, a_done, b_started = [], threading.Event(), threading.Event()

    def thread_a():
        try:
            sA = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(sA):
                gs.gs_unscale_check(gA, oA, SA, fA)     # caches the list
                sA.synchronize()
                fA.zero_()
                b_started.wait(30)
                R = oracle.ScalerState(2.0 ** 20)
                for cap in range(6):
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph, stream=sA, capture_error_mode="thread_local"):
                        gs.gs_unscale_check(gA, oA, SA, fA)
                        gs.gs_update_scale(SA, trA, fA, 2.0, 0.5, 3)
                    for r in range(3):
                        for out in oA:
                            out.fill_(-2.0)
                        graph.replay()
                        ref, rf = oracle.unscale_check(hA, float(R.S))
                        R.found_inf.value = rf
                        oracle.update_scale(R, 2.0, 0.5, 3)
                        sA.synchronize()
                        for out, rr in zip(oA, ref):
                            assert np.array_equal(_bits(out), rr.view(np.uint32)), (cap, r)
                        assert float(SA.item()) == float(R.S), (cap, r)
        except Exception as e:          # noqa: BLE001 -- reported below
            errors.append(("A", repr(e)))
        finally:
            a_done.set()

    def thread_b():
        try:
            sB = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(sB):
                k = 0
                while k < len(listsB) and (k < 100 or not a_done.is_set()):
                    host, g, o = listsB[k]
                    gs.gs_unscale_check(g, o, SB, fB[k])
                    b_started.set()
                    ref, rf = oracle.unscale_check(host, 128.0)
                    sB.synchronize()
                    for out, rr in zip(o, ref):
                        assert np.array_equal(_bits(out), rr.view(np.uint32)), k
                    assert int(fB[k].item()) == rf, k
                    k += 1
        except Exception as e:          # noqa: BLE001 -- reported below
            errors.append(("B", repr(e)))
        finally:
            b_started.set()

    ta, tb = threading.Thread(target=thread_a), threading.Thread(target=thread_b)
    ta.start()
    tb.start()
    ta.join()
    tb.join()
    assert not errors, errors
