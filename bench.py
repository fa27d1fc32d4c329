#!/usr/bin/env python3
"""Throughput of the loss-scaling + FP8 hot path on one MI355X.

One step = the whole path over one batch of synthetic, HBM-resident input:
  1. gs_unscale_check over a Llama-3-8B-shaped FP16 gradient set (291 tensors,
     8,030,261,248 elements, S = 2^15) -> FP32, one launch;
  2. gs_update_scale (device-resident state; Inf planted in lm_head on step 2);
  3. fp8_quantize of DeepSeek-V3-shaped BF16 activations 16384x7168 (1x128,
     E4M3) and weights 7168x18432 (128x128, E4M3), scales from the block amax;
  4. fp8_dequantize of both back to FP32.
value = algorithmic bytes of the step (every input read once, every output
written once) / wall time per step.  The unscale's kernel time comes from HIP
events on the launch stream inside the timed region (the only events there);
the other kernels' times from the same steps run again after it, untimed,
with events around every launch.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--no-cpu-baseline]
                    [--no-ceilings] [--all-configs]

After the step, `ceilings` gives the best rate of each access pattern the
kernels use (read, write, 2 B -> 4 B, 2 B -> 1 B, 1 B -> 4 B) at the
kernels' own sizes, from the streaming kernels of libgsceil.so, and every
kernel's `frac_of_ceiling` against its pattern.

Prints one JSON line.  More than one GPU is not supported (this path is
measured on one GPU; see the sharding notes in the design document).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for FP8 block quantize and fused unscale+inf-check"
PEAK_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "unscale_check_llama3_8b_pmc.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(files):
    """First 16 hex digits of the sha256 of the kernel sources' code: comments
    and whitespace are removed first, so that editing prose does not detach
    the committed counters from the kernel they were taken on."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "loss_scaling_fp8_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def pmc_traffic(src_hash):
    """HBM bytes per unscale launch from the committed rocprofv3 --pmc
    summary, or None when it is missing or was taken on other kernel source."""
    if not os.path.exists(PMC_FILE):
        return None
    vals = {}
    for line in open(PMC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_share():
    """(threads, host_cores, quota_cores): the cores in this process's
    affinity mask, limited by the cgroup CPU quota and by OMP_NUM_THREADS
    when either is set -- the CPU share a job on a shared GPU host is given
    (more threads than that only queue for the same cores)."""
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:
        host = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            q, period = fh.read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    threads = host
    if quota is not None:
        threads = min(threads, quota)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    return max(1, threads), host, quota


def cpu_baseline(grad_sample, act_rows, wgt_rows):
    """The oracle (plain C, untouched) on a bounded sample of the same
    workload, inputs being host copies of the device tensors: once on one
    core, then with the sample split into independent pieces (gradient
    chunks; activation row groups; 128-row weight groups, so no block is
    split) run by a thread pool over the host's cores (the C calls release
    the GIL), three times.  The median of the all-cores runs is the value."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle

    grad_pieces = np.array_split(grad_sample, 64)
    act_pieces = np.array_split(act_rows, 64)
    wgt_pieces = [wgt_rows[r:r + 128] for r in range(0, wgt_rows.shape[0], 128)]

    def unscale(g):
        oracle.unscale_check([g], 32768.0)

    def quant(x, gran):
        codes, scales, _ = oracle.quantize(x, 0, gran)
        oracle.dequantize(codes, 0, gran, scales)

    nbytes = grad_sample.size * 6
    for x, nb in ((act_rows, 128), (wgt_rows, 128 * 128)):
        nbytes += x.size * 8 + 2 * (x.size // nb) * 4
    jobs = [(unscale, (g,)) for g in grad_pieces] + [(quant, (x, 1)) for x in act_pieces] + \
           [(quant, (x, 2)) for x in wgt_pieces]
    t0 = time.perf_counter()
    for fn, a in jobs:
        fn(*a)
    t_one = time.perf_counter() - t0
    threads, host_cores, quota = cpu_share()
    runs = []
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(lambda j: j[0](*j[1]), jobs))
            runs.append(time.perf_counter() - t0)
    t_all = float(np.median(runs))
    return {"value": round(nbytes / t_all / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "value_1_core": round(nbytes / t_one / 1e9, 4),
            "host_cores": host_cores, "cgroup_cpu_quota": quota,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": "%d FP16 elements (embedding + lm_head gradients) unscaled, %dx%d "
                      "activation rows 1x128 and %dx%d weight rows 128x128 quantized and "
                      "dequantized, E4M3; the C oracle on %d threads (median of 3 runs, "
                      "%.1f s) and on 1 (%.1f s); %d cores in the affinity mask, the "
                      "threads limited to this job's CPU share (cgroup quota, "
                      "OMP_NUM_THREADS)"
                      % (grad_sample.size, act_rows.shape[0], act_rows.shape[1],
                         wgt_rows.shape[0], wgt_rows.shape[1], threads, t_all, t_one,
                         host_cores)}


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence:
    recording one then skips the system-scope release (a write-back of the
    caches) that a default event performs, which would otherwise be charged
    to the interval it bounds and to the step.  The HIP runtime is the one
    torch already loaded (same soname, so the same instance and streams).
    Elapsed times are read only after a device synchronisation."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        P = ctypes.c_void_p
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [P, P]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.hip.hipEventDestroy.argtypes = [P]
        self.events = []

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s returned %d" % (what, rc))

    def new(self):
        e = self.ct.c_void_p()
        self._ok(self.hip.hipEventCreateWithFlags(self.ct.byref(e), 0x20000000),
                 "hipEventCreateWithFlags(hipEventDisableSystemFence)")
        self.events.append(e)
        return e

    def record(self, e, stream):
        self._ok(self.hip.hipEventRecord(e, self.ct.c_void_p(stream)), "hipEventRecord")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)

    def destroy(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


CEIL_LIB = os.path.join(ROOT, "loss_scaling_fp8_amd", "libgsceil.so")
CEIL_PATTERNS = {"read": 0, "write": 1, "expand_2to4": 2, "narrow_2to1": 3, "expand_1to4": 4,
                 "expand_1to2": 5}
# bytes read and written by one pass of a pattern over n elements (read /
# write: n bytes)
CEIL_SRC_BYTES = {0: lambda n: n, 1: lambda n: 0, 2: lambda n: 2 * n, 3: lambda n: 2 * n,
                  4: lambda n: n, 5: lambda n: n}
CEIL_DST_BYTES = {0: lambda n: 0, 1: lambda n: n, 2: lambda n: 4 * n, 3: lambda n: n,
                  4: lambda n: 4 * n, 5: lambda n: 2 * n}
CEIL_POLICY = ("plain", "nt", "sc1nt")


def measure_ceilings(dev, specs, tev, reps=5):
    """Best sustained rate of each access pattern over a sweep of launch
    shapes, from the streaming kernels of libgsceil.so on flat buffers of
    the given sizes.  specs: (name, pattern, n) with n elements (read /
    write: bytes).  Launches run back to back, each between two HIP events
    on the current stream (the events of the unscale's own timing), so each
    pays for the previous launch's write drain, as the step's kernels do.  A
    working set below 4 GiB would partly stay in the 256 MB infinity cache
    and its writes drain after its end event, so such a pattern cycles
    through k buffer sets (k x working set >= 4 GiB): every launch reads
    from HBM.  Each variant: one untimed round over the sets, then
    max(reps, k) timed launches; the median is its time, the fastest
    variant the ceiling."""
    import ctypes

    import numpy as np
    import torch
    L = ctypes.CDLL(CEIL_LIB)
    L.gsc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p]
    L.gsc_stream.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, pattern, n in specs:
        p = CEIL_PATTERNS[pattern]
        src_bytes = CEIL_SRC_BYTES[p](n)
        dst_bytes = CEIL_DST_BYTES[p](n) if p else 1024
        work = src_bytes + dst_bytes
        k = max(1, min(16, -(-(4 << 30) // work)))
        sets = [(torch.empty(max(src_bytes, 16), dtype=torch.uint8, device=dev),
                 torch.empty(dst_bytes, dtype=torch.uint8, device=dev)) for _ in range(k)]
        moved = src_bytes + (0 if p == 0 else dst_bytes)
        best = None
        shapes = [(1, 0)] + [(u, lay) for u in (2, 4, 8) for lay in (0, 1)]
        for unroll, layout in shapes:
            for ntl in (0, 1):
                if p == 1 and ntl:
                    continue                       # no loads to vary
                for policy in range(3):
                    if p == 0 and policy:
                        continue                   # no stores to vary
                    for occ in (0, 7, 5):
                        args = [(p, s.data_ptr(), d.data_ptr(), n, unroll, layout, ntl, policy,
                                 occ, stream) for s, d in sets]
                        for a in args:
                            rc = L.gsc_stream(*a)
                            if rc != 0:
                                raise RuntimeError("gsc_stream%r returned %d" % (a[:1] + a[3:9], rc))
                        evs = [(tev.new(), tev.new()) for _ in range(max(reps, k))]
                        for j, (a, b) in enumerate(evs):
                            tev.record(a, stream)
                            L.gsc_stream(*args[j % k])
                            tev.record(b, stream)
                        torch.cuda.synchronize()
                        ms = float(np.median([tev.elapsed_ms(a, b) for a, b in evs]))
                        if best is None or ms < best[0]:
                            best = (ms, unroll, layout, ntl, policy, occ)
        ms, unroll, layout, ntl, policy, occ = best
        out[name] = {"GBps": round(moved / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4),
                     "bytes": moved, "elements": n, "pattern": pattern, "buffer_sets": k,
                     "variant": "unroll %d (%s), %s loads, %s stores, %s" % (
                         unroll, "lane-contiguous units" if layout else "wave-contiguous units",
                         "non-temporal" if ntl else "plain", CEIL_POLICY[policy],
                         "no occupancy cap" if occ == 0 else "%d workgroups per CU" % occ)}
        log("ceiling %s: %.0f GB/s (%s)" % (name, out[name]["GBps"], out[name]["variant"]))
        del sets
        torch.cuda.empty_cache()
    return out


def _time_launches(fn, reps, flush=None):
    """Median and minimum milliseconds of fn() over reps launches, from HIP
    events recorded on the current stream around each launch; flush() (not
    timed) is enqueued before each.  Everything is enqueued before the one
    wait at the end, so the GPU is busy with earlier work while the host
    marshals each call and the events time the GPU work only (the first
    launch may include host latency; the median ignores it)."""
    import numpy as np
    import torch
    evs = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return float(np.median(ts)), float(np.min(ts))


def _ceil_lib():
    import ctypes
    L = ctypes.CDLL(CEIL_LIB)
    L.gsc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_void_p]
    L.gsc_stream.restype = ctypes.c_int
    return L


def _gsc_call(L, a):
    rc = L.gsc_stream(*a)
    if rc != 0:
        raise RuntimeError("gsc_stream%r returned %d" % (a[:1] + a[3:9], rc))


def _cold_best(L, p, src, dst, n, flush, reps, policies=(0, 1, 2)):
    """Best median (ms, args) over the variants of single cold launches of
    pattern p over n elements: unroll 1/2/4, both unit layouts, plain or
    non-temporal loads, the given store policies, no cap or 6 workgroups per
    CU."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    best = None
    for unroll in (1, 2, 4):
        for layout in (0, 1):
            for ntl in (0, 1):
                for policy in ((0,) if p == 0 else policies):
                    for occ in (0, 6):
                        a = (p, src.data_ptr(), dst.data_ptr(), n, unroll, layout, ntl, policy,
                             occ, stream)
                        _gsc_call(L, a)
                        ms, _ = _time_launches(lambda: _gsc_call(L, a), reps, flush)
                        if best is None or ms < best[0]:
                            best = (ms, a)
    return best


def cold_ceiling(dev, pattern, n, flush, policies=(0, 1, 2), reps=20):
    """The least time one cold launch of `pattern` over n elements takes on
    this GPU (milliseconds by HIP events), with its bytes moved: the best of
    the streaming kernel's variants with the given store policies, each timed
    after flush().  A cold launch with plain (write-back) stores can end
    with part of its output still in the caches, so a write-heavy kernel is
    compared with the ceiling of its own store class."""
    import torch
    L = _ceil_lib()
    p = CEIL_PATTERNS[pattern]
    src = torch.zeros(max(CEIL_SRC_BYTES[p](n), 16), dtype=torch.uint8, device=dev)
    dst = torch.empty(max(CEIL_DST_BYTES[p](n), 1024), dtype=torch.uint8, device=dev)
    ms, a = _cold_best(L, p, src, dst, n, flush, reps, policies)
    del src, dst
    unroll, layout, ntl, policy, occ = a[4:9]
    return {"ms": round(ms, 4), "bytes": CEIL_SRC_BYTES[p](n) + CEIL_DST_BYTES[p](n),
            "pattern": pattern,
            "variant": "unroll %d (%s), %s loads, %s stores, %s" % (
                unroll, "lane-contiguous units" if layout else "wave-contiguous units",
                "non-temporal" if ntl else "plain", CEIL_POLICY[policy],
                "no occupancy cap" if occ == 0 else "%d workgroups per CU" % occ)}


def cold_two_pass_ceiling(dev, n, flush, reps=20):
    """The least a two-pass per-tensor quantize of n BF16 elements can take on
    this GPU, from the streaming kernels: the best variant of a cold read of
    the 2n input bytes, the best variant of a cold 2 B -> 1 B stream over the
    same buffer, then the two launched back to back after a flush (the
    amax-then-cast sequence, with the second read finding what the first
    left in the caches).  Milliseconds by HIP events, medians of reps."""
    import torch
    L = _ceil_lib()
    src = torch.zeros(2 * n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.empty(1024, dtype=torch.uint8, device=dev)
    rd = _cold_best(L, 0, src, sink, 2 * n, flush, reps)
    nw = _cold_best(L, 3, src, dst, n, flush, reps)
    seq, _ = _time_launches(lambda: (_gsc_call(L, rd[1]), _gsc_call(L, nw[1])), reps, flush)
    del src, dst, sink
    return {"read_ms": round(rd[0], 4), "narrow_2to1_ms": round(nw[0], 4),
            "read_then_narrow_ms": round(seq, 4),
            "note": "streaming kernels on the same sizes, cold; best of 24 read and 72 "
                    "2 B -> 1 B variants, then the best two back to back"}


def measure_configs(dev):
    """Per-configuration kernel timings outside the step: the tiny case, the
    8192x8192 per-tensor pair and the 4 GiB special-value tensors.  A 1 GiB
    write and a 1 GiB read evict the 256 MB infinity cache before each timed
    launch of the per-tensor pair."""
    import torch

    import loss_scaling_fp8_amd as gs
    import synth

    junk = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    junk_rd = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        # a 1 GiB write then a 1 GiB read (stream-ordered): a cold cache that
        # holds clean lines, so no write-back is charged to the timed launch
        junk.fill_(1.0)
        junk_rd.sum()

    res = {}
    # tiny: 16 FP16 tensors (2^20 elements) unscale + update; 1024^2 per-tensor E4M3
    g = synth.tiny_gradset()
    grads = [g.full(t, dev) for t in range(len(g.tensors))]
    outs = [torch.empty(sp.numel, dtype=torch.float32, device=dev) for sp in g.tensors]
    S = torch.tensor([g.scale], device=dev)
    tr = torch.zeros(1, dtype=torch.int32, device=dev)
    fi = torch.zeros(1, dtype=torch.int32, device=dev)
    gs.gs_unscale_check(grads, outs, S, fi)
    torch.cuda.synchronize()
    ms, _ = _time_launches(lambda: (gs.gs_unscale_check(grads, outs, S, fi),
                                    gs.gs_update_scale(S, tr, fi, 2.0, 0.5, 2000)), 50)
    # the same step captured in a HIP graph (the list is cached, so the
    # calls allocate nothing): one replay per step removes the host launch cost
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gs.gs_unscale_check(grads, outs, S, fi)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        gs.gs_unscale_check(grads, outs, S, fi)
        gs.gs_update_scale(S, tr, fi, 2.0, 0.5, 2000)
    graph.replay()
    torch.cuda.synchronize()
    ms_graph, _ = _time_launches(graph.replay, 50)
    q = synth.tiny_quant()
    xq = q.full(dev)
    cq, sq = gs.fp8_quantize(xq, q.fmt, q.gran)
    ms_q, _ = _time_launches(lambda: gs.fp8_quantize(xq, q.fmt, q.gran, 0, cq, sq), 50)
    dq = gs.fp8_dequantize(cq, q.fmt, q.gran, sq)
    ms_d, _ = _time_launches(lambda: gs.fp8_dequantize(cq, q.fmt, q.gran, sq, dq), 50)
    res["tiny"] = {"unscale+update_us_per_step": round(ms * 1e3, 2),
                   "unscale+update_us_per_step_hip_graph": round(ms_graph * 1e3, 2),
                   "quant_per_tensor_1024x1024_us": round(ms_q * 1e3, 2),
                   "dequant_1024x1024_us": round(ms_d * 1e3, 2),
                   "note": "launch-bound and cache-resident: correctness case, no GB/s claim"}
    del grads, outs
    # per-tensor at scale
    pt = {}
    specs = synth.per_tensor_at_scale()
    ceil = cold_two_pass_ceiling(dev, specs[0].rows * specs[0].cols, flush)
    pt["two_pass_ceiling"] = ceil
    for sp in specs:
        x = sp.full(dev)
        n = sp.rows * sp.cols
        codes, scales = gs.fp8_quantize(x, sp.fmt, sp.gran)
        ws = torch.empty(gs.fp8_quantize_workspace_size(sp.rows, sp.cols, sp.gran),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((sp.rows, sp.cols), dtype=torch.float32, device=dev)
        mq, mq_min = _time_launches(lambda: gs.fp8_quantize(x, sp.fmt, sp.gran, 0, codes, scales,
                                                            None, ws), 20, flush)
        md, _ = _time_launches(lambda: gs.fp8_dequantize(codes, sp.fmt, sp.gran, scales, out),
                               20, flush)
        st = torch.ones(1, dtype=torch.float32, device=dev)
        hist = torch.zeros(16, dtype=torch.float32, device=dev)
        pos = torch.zeros(1, dtype=torch.int32, device=dev)
        used = torch.empty(1, dtype=torch.float32, device=dev)
        mdl, _ = _time_launches(lambda: gs.fp8_quantize_delayed(x, sp.fmt, st, hist, pos, codes,
                                                                used, None, ws), 20, flush)
        bq, bd = n * 3 + 4, n * 5 + 4
        pt[sp.name] = {"quant_ms": round(mq, 4), "quant_GBps": round(bq / mq / 1e6, 1),
                       "quant_hbm_GBps_with_reread": round((bq + 2 * n) / mq / 1e6, 1),
                       "quant_frac_of_two_pass_ceiling":
                           round(ceil["read_then_narrow_ms"] / mq, 3),
                       "delayed_quant_ms": round(mdl, 4),
                       "delayed_quant_GBps": round(bq / mdl / 1e6, 1),
                       "dequant_ms": round(md, 4), "dequant_GBps": round(bd / md / 1e6, 1)}
        del x, codes, scales, out
    res["per_tensor_8192"] = pt
    # 4 GiB special values, scales from the block amax
    tev = TimingEvents()
    sv = measure_special_values(dev, [sp.name for sp in synth.special_values_4gib()],
                                ("e4m3", "e5m2"), ("cold", "b2b"), 20, tev)
    tev.destroy()
    res["special_4gib"] = sv
    return res


def measure_special_values(dev, tensors, fmts, phases, reps, tev=None):
    """The four 16384x32768 BF16 special-value tensors: quantize with scales
    from the amax (per-tensor, 1x128, 128x128) and the FP32 dequantize, per
    tensor x format x granularity, `reps` launches each.  Phase "cold": a
    1 GiB write and a 1 GiB read (stream-ordered, untimed) before every
    launch, so that the previous launch's writes have drained and the cache
    holds clean lines of other data; phase "b2b": the launches back to back,
    each paying for the previous one's write drain.  Medians of HIP-event
    times; GB/s from the algorithmic bytes.  With `tev` (TimingEvents), the
    sustained ceilings of the 2 B -> 1 B and 1 B -> 4 B patterns at this
    size are measured too, and each block-granularity entry gets its
    fraction of them."""
    import torch

    import loss_scaling_fp8_amd as gs
    import synth

    junk = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    junk_rd = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        junk.fill_(1.0)
        junk_rd.sum()

    fmt_id = {"e4m3": gs.FP8_E4M3, "e5m2": gs.FP8_E5M2}
    grans = ((gs.FP8_PER_TENSOR, "tensor"), (gs.FP8_BLOCK_1x128, "1x128"),
             (gs.FP8_BLOCK_128x128, "128x128"))
    sv = {}
    for sp in synth.special_values_4gib():
        if sp.name not in tensors:
            continue
        x = sp.full(dev)
        n = sp.rows * sp.cols
        codes = torch.empty((sp.rows, sp.cols), dtype=torch.uint8, device=dev)
        out = torch.empty((sp.rows, sp.cols), dtype=torch.float32, device=dev)
        ws = torch.empty(gs.fp8_quantize_workspace_size(sp.rows, sp.cols, gs.FP8_PER_TENSOR),
                         dtype=torch.uint8, device=dev)
        for fname in fmts:
            fmt = fmt_id[fname]
            for gran, gname in grans:
                sc = torch.empty(gs.scale_shape(sp.rows, sp.cols, gran), dtype=torch.float32,
                                 device=dev)
                gs.fp8_quantize(x, fmt, gran, 0, codes, sc, None, ws)
                ns = sc.numel()
                bq, bd = n * 3 + ns * 4, n * 5 + ns * 4
                for phase in phases:
                    fl = flush if phase == "cold" else None
                    mq, mq_min = _time_launches(
                        lambda: gs.fp8_quantize(x, fmt, gran, 0, codes, sc, None, ws), reps, fl)
                    md, md_min = _time_launches(
                        lambda: gs.fp8_dequantize(codes, fmt, gran, sc, out), reps, fl)
                    key = "%s/%s/%s/%s" % (sp.name, fname, gname, phase)
                    sv[key] = {"quant_ms": round(mq, 4), "quant_GBps": round(bq / mq / 1e6, 1),
                               "quant_GBps_best": round(bq / mq_min / 1e6, 1),
                               "dequant_ms": round(md, 4),
                               "dequant_GBps": round(bd / md / 1e6, 1),
                               "dequant_GBps_best": round(bd / md_min / 1e6, 1)}
                    log("%s: quant %.0f GB/s, dequant %.0f GB/s" %
                        (key, sv[key]["quant_GBps"], sv[key]["dequant_GBps"]))
                del sc
        del x, codes, out
        torch.cuda.empty_cache()
    sv["note"] = ("per-tensor runs two passes over the input (amax, then cast): its GB/s "
                  "counts the algorithmic 3 B/element, the traffic is 5 B/element")
    if tev is not None:
        n = synth.special_values_4gib()[0].rows * synth.special_values_4gib()[0].cols
        ceil = measure_ceilings(dev, [("narrow_2to1", "narrow_2to1", n),
                                      ("expand_1to4", "expand_1to4", n)], tev)
        for key, e in sv.items():
            if key != "note" and "/tensor/" not in key:
                e["quant_frac_of_ceiling"] = round(e["quant_GBps"] / ceil["narrow_2to1"]["GBps"], 4)
                e["dequant_frac_of_ceiling"] = round(e["dequant_GBps"] / ceil["expand_1to4"]["GBps"], 4)
        sv["ceilings"] = ceil
    return sv


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-kernel ceilings (about 5 s)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time the tiny, per-tensor 8192^2 and 4 GiB special-value "
                         "configurations (reported under \"configs\")")
    ap.add_argument("--special-values", nargs=3, metavar=("TENSOR", "FMT", "PHASE"),
                    help="only time the 4 GiB special-value quantize/dequantize for one "
                         "tensor (mix, anchored, saturation, random), format (e4m3, e5m2, "
                         "both) and phase (cold, b2b), 20 launches each (for per-configuration "
                         "kernel-trace profiles); prints one JSON object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 6 plain copy kernels of 1 GiB (for HBM counter calibration)")
    ap.add_argument("--extensions", "--sumsq", dest="extensions", action="store_true",
                    help="with --pmc-safe: also run the launches outside the step (unscale + "
                         "sum of squares, 1x32 and MX blocks)")
    ap.add_argument("--pmc-safe", action="store_true",
                    help="for rocprofv3 --pmc runs: constant inputs (few kernel launches), no "
                         "device-to-device or device-to-host memcpy, no copy ceiling, no "
                         "final-state readback, no CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU path only: --gpus must be 1 (sharding across "
              "GPUs is described in the design notes and not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import loss_scaling_fp8_amd as gs
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.special_values:
        t, f, ph = args.special_values
        if t not in ("mix", "anchored", "saturation", "random") or \
                f not in ("e4m3", "e5m2", "both") or ph not in ("cold", "b2b"):
            ap.error("--special-values TENSOR FMT PHASE: see --help")
        gs.lib()
        fmts = ("e4m3", "e5m2") if f == "both" else (f,)
        tev = None if args.no_ceilings else TimingEvents()
        sv = measure_special_values(dev, (t,), fmts, (ph,), 20, tev)
        if tev is not None:
            tev.destroy()
        print(json.dumps({"special_4gib": sv}))
        return
    if args.copy_calibration:
        # int32 -> float32 converting copy: an elementwise kernel reading and
        # writing 4 bytes per element (a same-type copy would be a memcpy)
        a = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
        b = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(6):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": {"read": a.numel() * 4,
                                                                "write": b.numel() * 4}}))
        return
    gs.lib()

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    gset = synth.llama3_8b_gradset()
    grads, outs = [], []
    for t, sp in enumerate(gset.tensors):
        if args.pmc_safe:
            # counter runs: constant inputs, one fill kernel per tensor (HBM
            # traffic does not depend on the values)
            grads.append(torch.empty(sp.numel, dtype=torch.float16, device=dev).fill_(0.5))
        else:
            grads.append(gset.full(t, dev))
        outs.append(torch.empty(sp.numel, dtype=torch.float32, device=dev))
        if t % 40 == 0:
            log("generated gradient %d/%d (%.0f s)" % (t + 1, len(gset.tensors), time.time() - t0))
    act, wgt = synth.deepseek_v3_blocks()
    if args.pmc_safe:
        xa = torch.empty((act.rows, act.cols), dtype=torch.bfloat16, device=dev).fill_(0.5)
        xw = torch.empty((wgt.rows, wgt.cols), dtype=torch.bfloat16, device=dev).fill_(0.5)
    else:
        xa, xw = act.full(dev), wgt.full(dev)
    ca = torch.empty((act.rows, act.cols), dtype=torch.uint8, device=dev)
    cw = torch.empty((wgt.rows, wgt.cols), dtype=torch.uint8, device=dev)
    sa = torch.empty(gs.scale_shape(act.rows, act.cols, act.gran), dtype=torch.float32, device=dev)
    sw = torch.empty(gs.scale_shape(wgt.rows, wgt.cols, wgt.gran), dtype=torch.float32, device=dev)
    da = torch.empty((act.rows, act.cols), dtype=torch.float32, device=dev)
    dw = torch.empty((wgt.rows, wgt.cols), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs resident in HBM (%.0f s)" % (time.time() - t0))

    S = torch.empty(1, dtype=torch.float32, device=dev)
    tracker = torch.empty(1, dtype=torch.int32, device=dev)
    found = torch.empty(1, dtype=torch.int32, device=dev)
    skips = torch.empty(1, dtype=torch.int64, device=dev)

    def reset_state():
        S.fill_(gset.scale)
        tracker.zero_()
        found.zero_()
        skips.zero_()

    inj_t, inj_i, _ = gset.injections[2][0]
    inj_slot = grads[inj_t][inj_i:inj_i + 1]
    inj_orig = float(synth.to_f16_tensor(gset.gen(inj_t, torch.tensor([inj_i]))).float()[0])

    n_grad = gset.total
    n_a, n_w = act.rows * act.cols, wgt.rows * wgt.cols
    ns_a, ns_w = sa.numel(), sw.numel()
    bytes_unscale = n_grad * (2 + 4)
    bytes_qa = n_a * 3 + ns_a * 4
    bytes_qw = n_w * 3 + ns_w * 4
    bytes_da = n_a * 5 + ns_a * 4
    bytes_dw = n_w * 5 + ns_w * 4
    bytes_update = 4 + 4 + 4 + 8 + 4 + 4 + 4 + 8
    step_bytes = bytes_unscale + bytes_update + bytes_qa + bytes_qw + bytes_da + bytes_dw

    names = ["unscale_check", "update_scale", "quant_1x128", "quant_128x128",
             "dequant_1x128", "dequant_128x128"]

    stream_handle = torch.cuda.current_stream().cuda_stream
    tev = TimingEvents()

    def step(k, ev):
        if k == 2:
            inj_slot.fill_(float("inf"))
        calls = [
            lambda: gs.gs_unscale_check(grads, outs, S, found),
            lambda: gs.gs_update_scale(S, tracker, found, 2.0, 0.5, 2000, skips),
            lambda: gs.fp8_quantize(xa, act.fmt, act.gran, gs.FP8_SCALE_FROM_AMAX, ca, sa),
            lambda: gs.fp8_quantize(xw, wgt.fmt, wgt.gran, gs.FP8_SCALE_FROM_AMAX, cw, sw),
            lambda: gs.fp8_dequantize(ca, act.fmt, act.gran, sa, da),
            lambda: gs.fp8_dequantize(cw, wgt.fmt, wgt.gran, sw, dw),
        ]
        for j, c in enumerate(calls):
            if ev is not None and ev[j] is not None:
                tev.record(ev[j][0], stream_handle)
            c()
            if ev is not None and ev[j] is not None:
                tev.record(ev[j][1], stream_handle)
        if k == 2:
            inj_slot.fill_(inj_orig)

    reset_state()
    for w in range(args.warmup):
        step(w + 1, None)
    torch.cuda.synchronize()
    log("warmup done")
    def new_events(which):
        return [[[tev.new(), tev.new()] if j in which else None for j in range(len(names))]
                for _ in range(args.steps)]

    def mean_ms(events, j):
        return float(np.mean([tev.elapsed_ms(events[k][j][0], events[k][j][1])
                              for k in range(args.steps)]))

    # timed steps: HIP events (without the system-scope fence) bracket the
    # dominant kernel, the unscale, only; an event pair around every launch
    # costs about 0.5% of the step
    reset_state()
    events = new_events({0})
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(1, args.steps + 1):
        step(k, events[k - 1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    log("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step))
    state = (None, None, None)
    if not args.pmc_safe:
        state = (float(S.item()), int(tracker.item()), int(skips.item()))
        log("final S=%g tracker=%d skips=%d" % state)
    # per-kernel breakdown: the same steps again, untimed, with events around
    # every launch (the unscale's figure stays the timed steps' own)
    per_kernel_ms = {names[0]: mean_ms(events, 0)}
    reset_state()
    events_all = new_events(set(range(len(names))))
    for k in range(1, args.steps + 1):
        step(k, events_all[k - 1])
    torch.cuda.synchronize()
    for j, n in enumerate(names[1:], 1):
        per_kernel_ms[n] = mean_ms(events_all, j)
    ceilings = None
    if not args.pmc_safe and not args.no_ceilings:
        # achievable rate of each access pattern at the kernels' own sizes
        # (flat buffers, outside the step; about 50 GB more of HBM)
        ceilings = measure_ceilings(dev, [
            ("read", "read", n_grad * 2), ("write", "write", n_grad * 4),
            ("expand_2to4", "expand_2to4", n_grad),
            ("narrow_2to1_act", "narrow_2to1", n_a), ("narrow_2to1_wgt", "narrow_2to1", n_w),
            ("expand_1to4_act", "expand_1to4", n_a), ("expand_1to4_wgt", "expand_1to4", n_w)],
            tev)
    tev.destroy()

    kbytes = {"unscale_check": bytes_unscale, "update_scale": bytes_update,
              "quant_1x128": bytes_qa, "quant_128x128": bytes_qw,
              "dequant_1x128": bytes_da, "dequant_128x128": bytes_dw}
    kceil = {"unscale_check": "expand_2to4", "quant_1x128": "narrow_2to1_act",
             "quant_128x128": "narrow_2to1_wgt", "dequant_1x128": "expand_1to4_act",
             "dequant_128x128": "expand_1to4_wgt"}
    kernels = {}
    for n in names:
        gbps = kbytes[n] / (per_kernel_ms[n] * 1e-3) / 1e9
        kernels[n] = {"ms": round(per_kernel_ms[n], 4), "bytes": kbytes[n],
                      "GBps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4)}
        if ceilings and n in kceil:
            kernels[n]["ceiling"] = kceil[n]
            kernels[n]["frac_of_ceiling"] = round(gbps / ceilings[kceil[n]]["GBps"], 4)

    # unscale fused with the exact gradient sum of squares, on the same
    # resident gradient set (outside the timed step; own HIP events)
    ext = {}
    if not args.pmc_safe or args.extensions:
        acc = torch.zeros(2, dtype=torch.int64, device=dev)
        nsq = torch.empty(1, dtype=torch.float64, device=dev)
        ws = torch.empty(gs.gs_unscale_check_sumsq_workspace_size([g.numel() for g in grads]),
                         dtype=torch.uint8, device=dev)
        S.fill_(gset.scale)
        found.zero_()
        gs.gs_unscale_check_sumsq(grads, outs, S, found, acc, nsq, ws)
        ms_sq, ms_sq_min = _time_launches(
            lambda: gs.gs_unscale_check_sumsq(grads, outs, S, found, acc, nsq, ws), 10)
        gbps = bytes_unscale / (ms_sq * 1e-3) / 1e9
        ext["unscale_check_sumsq"] = {
            "ms": round(ms_sq, 4), "bytes": bytes_unscale, "GBps": round(gbps, 1),
            "frac_of_peak": round(gbps / PEAK_GBPS, 4),
            "vs_unscale_check": round(per_kernel_ms["unscale_check"] / ms_sq, 4),
            "note": "three launches (unscale + per-chunk partials, 128-bit reduction, final); "
                    "bytes count the FP16 read and FP32 write only"}
        log("unscale+sumsq: %.3f ms (%.0f GB/s)" % (ms_sq, gbps))
        del ws

    # 1x32 blocks (FP32 scales, and MX-style E8M0 scales) on the activation
    # shape, outside the timed step, with the 1x128 pair timed the same way
    # for reference.  Before each timed launch a 1 GiB write and then a 1 GiB
    # read (stream-ordered) leave the infinity cache holding clean lines of
    # other buffers: cold inputs, and no write-back of an unrelated kernel's
    # dirty lines charged to the launch.
    if not args.pmc_safe or args.extensions:
        junk = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        junk_rd = torch.ones(1 << 28, dtype=torch.float32, device=dev)

        def flush():
            junk.fill_(1.0)
            junk_rd.sum()
        s32 = torch.empty(gs.scale_shape(act.rows, act.cols, gs.FP8_BLOCK_1x32),
                          dtype=torch.float32, device=dev)
        smx = torch.empty((act.rows, act.cols // 32), dtype=torch.uint8, device=dev)
        nb32, nb128 = n_a // 32, n_a // 128
        da_bf = torch.empty((act.rows, act.cols), dtype=torch.bfloat16, device=dev)
        dw_bf = torch.empty((wgt.rows, wgt.cols), dtype=torch.bfloat16, device=dev)
        act_wl = "%dx%d bf16 E4M3, cold (clean) infinity cache" % (act.rows, act.cols)
        wgt_wl = "%dx%d bf16 E4M3 128x128, cold (clean) infinity cache" % (wgt.rows, wgt.cols)
        # the same patterns streamed cold by the ceiling kernels, one launch
        # after the same flush: what a single cold launch of that size can reach
        cold = {}
        if not args.pmc_safe and not args.no_ceilings:
            # the quantizers store codes with plain stores, the dequantizers
            # their outputs with non-temporal ones: each is compared with the
            # streaming kernel restricted to the same store class
            for cname, pat, ne, pol in (("narrow_2to1_act", "narrow_2to1", n_a, (0,)),
                                        ("expand_1to4_act", "expand_1to4", n_a, (1, 2)),
                                        ("expand_1to2_act", "expand_1to2", n_a, (1, 2)),
                                        ("expand_1to2_wgt", "expand_1to2", n_w, (1, 2))):
                cold[cname] = cold_ceiling(dev, pat, ne, flush, pol)
            ext["cold_ceilings"] = cold
        ext_ceil = {"quant_1x128_cold": "narrow_2to1_act", "quant_1x32": "narrow_2to1_act",
                    "quant_mx_e8m0": "narrow_2to1_act", "dequant_1x128_cold": "expand_1to4_act",
                    "dequant_1x32": "expand_1to4_act", "dequant_mx_e8m0": "expand_1to4_act",
                    "dequant_1x128_bf16": "expand_1to2_act",
                    "dequant_128x128_bf16": "expand_1to2_wgt"}
        for name, fn, nbytes, wl in (
                ("quant_1x128_cold", lambda: gs.fp8_quantize(xa, act.fmt, act.gran, 0, ca, sa),
                 n_a * 3 + nb128 * 4, act_wl),
                ("dequant_1x128_cold", lambda: gs.fp8_dequantize(ca, act.fmt, act.gran, sa, da),
                 n_a * 5 + nb128 * 4, act_wl),
                ("dequant_1x128_bf16", lambda: gs.fp8_dequantize_bf16(ca, act.fmt, act.gran, sa,
                                                                      da_bf),
                 n_a * 3 + nb128 * 4, act_wl),
                ("dequant_128x128_bf16", lambda: gs.fp8_dequantize_bf16(cw, wgt.fmt, wgt.gran, sw,
                                                                        dw_bf),
                 n_w * 3 + ns_w * 4, wgt_wl),
                ("quant_1x32", lambda: gs.fp8_quantize(xa, act.fmt, gs.FP8_BLOCK_1x32, 0, ca, s32),
                 n_a * 3 + nb32 * 4, act_wl),
                ("dequant_1x32", lambda: gs.fp8_dequantize(ca, act.fmt, gs.FP8_BLOCK_1x32, s32, da),
                 n_a * 5 + nb32 * 4, act_wl),
                ("quant_mx_e8m0", lambda: gs.fp8_quantize_mx(xa, act.fmt, ca, smx), n_a * 3 + nb32,
                 act_wl),
                ("dequant_mx_e8m0", lambda: gs.fp8_dequantize_mx(ca, act.fmt, smx, da),
                 n_a * 5 + nb32, act_wl)):
            fn()
            ms_k, _ = _time_launches(fn, 20, None if args.pmc_safe else flush)
            gbps = nbytes / (ms_k * 1e-3) / 1e9
            ext[name] = {"ms": round(ms_k, 4), "bytes": nbytes, "GBps": round(gbps, 1),
                         "frac_of_peak": round(gbps / PEAK_GBPS, 4), "workload": wl}
            c = cold.get(ext_ceil.get(name))
            if c:
                cg = c["bytes"] / (c["ms"] * 1e-3) / 1e9
                ext[name]["cold_ceiling"] = ext_ceil[name]
                ext[name]["frac_of_cold_ceiling"] = round(gbps / cg, 4)
        del junk, junk_rd, s32, smx, da_bf, dw_bf

    src_hash = kernel_source_hash(["unscale.hip", "gs_internal.hpp"])
    un = kernels["unscale_check"]
    roofline = {"bound": "hbm", "achieved": un["GBps"], "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(un["GBps"] / PEAK_GBPS, 4), "traffic": pmc_traffic(src_hash),
                "kernel": "unscale_check_kernel", "algorithmic_bytes_per_launch": bytes_unscale,
                "frac_of_ceiling": un.get("frac_of_ceiling")}

    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama3-8b fp16 grad set unscale+check+update (291 tensors, "
                               "8030261248 elems, S=2^15, Inf in lm_head at step 2) + "
                               "deepseek-v3 act 16384x7168 1x128 and wgt 7168x18432 128x128 "
                               "E4M3 quantize+dequantize",
                   "step_bytes": step_bytes, "grad_elems": n_grad,
                   "act_shape": [act.rows, act.cols], "wgt_shape": [wgt.rows, wgt.cols]},
        "roofline": roofline,
        "kernels": kernels,
        "extensions": ext,
        "ceilings": ceilings,
        "final_state": {"S": state[0], "tracker": state[1], "skips": state[2]},
    }
    if not args.no_cpu_baseline and not args.pmc_safe:
        log("cpu baseline (oracle) ...")
        g_host = np.concatenate([grads[0].view(-1).cpu().view(torch.int16).numpy(),
                                 grads[-1].view(-1).cpu().view(torch.int16).numpy()]).view(np.uint16)
        a_host = xa[:8192].cpu().view(torch.int16).numpy().view(np.uint16)
        w_host = xw[:2048].cpu().view(torch.int16).numpy().view(np.uint16)
        result["cpu_baseline"] = cpu_baseline(g_host, a_host, w_host)
    if args.all_configs:
        del grads, outs, xa, xw, da, dw
        torch.cuda.empty_cache()
        log("other configurations ...")
        result["configs"] = measure_configs(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
