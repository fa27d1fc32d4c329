// api.hip -- the C ABI of libgsfp8 (declared in include/gs.h): argument
// validation on the host, the cached per-chunk descriptors of the
// multi-tensor unscale, and dispatch to the kernels.  No entry point
// synchronises the device or reads device memory; device memory is taken
// only the first time a given gradient list is seen (its descriptors are
// cached, and that first call waits for their upload).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <list>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "gs.h"
#include "gs_internal.hpp"

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;

// ------------------------------------------------------------ work-list cache
// Key: device id + the (input, output, numel) triplets.  Value: a device
// buffer holding the per-chunk descriptors, and one event per stream that
// has launched a kernel reading it, re-recorded after every such launch.
// A caller enqueues its kernel while holding the cache lock (with_list), so
// no list can be evicted between its lookup and the launch that reads it.
//
// No call frees device memory or waits for the device (hipFree would
// synchronise the whole device, behind every other thread's queued work,
// and is not allowed while another thread captures a graph):
//  * the least recently used lists are evicted by count and by bytes.  An
//    evicted list's buffer is retired together with its events; a later
//    list takes it over (best fit, at most twice the size it needs) once
//    hipEventQuery reports every event complete.  Only when the retired
//    buffers of a device exceed kCacheBytes are the idle ones freed, which
//    happens when callers keep creating lists larger than any retired one;
//  * a list launched while its stream is capturing a graph is pinned: the
//    graph holds the descriptor address and may be replayed at any later
//    time, so that list is never evicted;
//  * uploads go through an internal non-blocking stream per device and wait
//    for that stream only.
struct DevBuffer {
    void *dev = nullptr;
    size_t cap = 0;
    int device = 0;
};

struct StreamUse {
    hipStream_t stream;
    hipEvent_t event;
};

struct CachedList {
    DevBuffer buf;
    int64_t nchunks = 0;
    bool pinned = false;
    std::vector<StreamUse> uses;
};

struct Retired {
    DevBuffer buf;
    std::vector<StreamUse> uses;
};

constexpr size_t kCacheEntries = 64;
constexpr size_t kCacheBytes = size_t(1) << 30;
constexpr size_t kBufferGranule = size_t(64) << 10;

struct ListCache {
    std::mutex mu;
    size_t bytes = 0;                          // capacity of the cached lists
    std::list<std::string> lru;                // front = most recent
    std::unordered_map<std::string, std::pair<CachedList, std::list<std::string>::iterator>> map;
    std::list<Retired> retired;                // front = most recently retired
    std::unordered_map<int, hipStream_t> upload_stream;
};

ListCache &cache() {
    static ListCache *c = new ListCache();   // never destroyed (no teardown-order issues)
    return *c;
}

std::string make_key(int device, int32_t n, const void *const *in, float *const *out,
                     const int64_t *numel) {
    std::string k;
    k.resize(sizeof(int) + size_t(n) * 3 * sizeof(uint64_t));
    char *p = &k[0];
    std::memcpy(p, &device, sizeof(int));
    p += sizeof(int);
    for (int32_t i = 0; i < n; ++i) {
        const uint64_t t[3] = {uint64_t(uintptr_t(in[i])), uint64_t(uintptr_t(out[i])),
                               uint64_t(numel[i])};
        std::memcpy(p, t, sizeof(t));
        p += sizeof(t);
    }
    return k;
}

// The chunk descriptors of a list, on the host (no HIP call).  GS_ERR_ARG
// when an address reaches 2^48.
gs_status make_descriptors(int32_t n, const void *const *in, float *const *out,
                           const int64_t *numel, std::vector<gsk::ChunkDesc> &host) {
    using gsk::kUnscaleChunk;
    int64_t total = 0;
    for (int32_t i = 0; i < n; ++i) total += (numel[i] + kUnscaleChunk - 1) / kUnscaleChunk;
    host.assign(static_cast<size_t>(total), gsk::ChunkDesc{0, 0});
    size_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (numel[i] == 0) continue;
        const uint64_t a_in = uint64_t(uintptr_t(in[i]));
        const uint64_t a_out = uint64_t(uintptr_t(out[i]));
        const uint64_t last_in = a_in + uint64_t(numel[i]) * 2;
        const uint64_t last_out = a_out + uint64_t(numel[i]) * 4;
        if (last_in > gsk::kAddrMask || last_out > gsk::kAddrMask) return GS_ERR_ARG;
        const uint64_t scalar = ((a_in | a_out) & 15u) ? 1u : 0u;
        for (int64_t st = 0; st < numel[i]; st += kUnscaleChunk) {
            const int64_t left = numel[i] - st;
            const uint64_t ragged = left < kUnscaleChunk ? uint64_t(left) : 0u;
            host[k].in_bits = (a_in + uint64_t(st) * 2) | (ragged << 48);
            host[k].out_bits = (a_out + uint64_t(st) * 4) | scalar;
            ++k;
        }
    }
    return GS_OK;
}

// True when every kernel that read the buffer has finished.
bool uses_done(const std::vector<StreamUse> &uses) {
    for (const StreamUse &u : uses)
        if (hipEventQuery(u.event) != hipSuccess) return false;
    return true;
}

void destroy_uses(std::vector<StreamUse> &uses) {
    for (StreamUse &u : uses) (void)hipEventDestroy(u.event);
    uses.clear();
}

// A buffer of at least `need` bytes on `device`: an idle retired one (best
// fit, at most twice the size), else a new allocation.
gs_status take_buffer(ListCache &c, int device, size_t need, DevBuffer &out) {
    auto best = c.retired.end();
    for (auto it = c.retired.begin(); it != c.retired.end(); ++it) {
        if (it->buf.device != device || it->buf.cap < need || it->buf.cap > 2 * need) continue;
        if (best != c.retired.end() && it->buf.cap >= best->buf.cap) continue;
        if (!uses_done(it->uses)) continue;
        best = it;
    }
    if (best != c.retired.end()) {
        out = best->buf;
        destroy_uses(best->uses);
        c.retired.erase(best);
        return GS_OK;
    }
    const size_t cap = (need + kBufferGranule - 1) / kBufferGranule * kBufferGranule;
    void *dev = nullptr;
    if (hipMalloc(&dev, cap) != hipSuccess) return GS_ERR_HIP;
    out = DevBuffer{dev, cap, device};
    return GS_OK;
}

gs_status upload_stream(ListCache &c, int device, hipStream_t *s) {
    auto it = c.upload_stream.find(device);
    if (it != c.upload_stream.end()) {
        *s = it->second;
        return GS_OK;
    }
    if (hipStreamCreateWithFlags(s, hipStreamNonBlocking) != hipSuccess) return GS_ERR_HIP;
    c.upload_stream.emplace(device, *s);
    return GS_OK;
}

gs_status build_list(ListCache &c, int device, int32_t n, const void *const *in,
                     float *const *out, const int64_t *numel, CachedList &cl) {
    std::vector<gsk::ChunkDesc> host;
    gs_status st = make_descriptors(n, in, out, numel, host);
    if (st != GS_OK) return st;
    const size_t bytes = host.size() * sizeof(gsk::ChunkDesc);
    hipStream_t up;
    st = upload_stream(c, device, &up);
    if (st != GS_OK) return st;
    DevBuffer buf;
    st = take_buffer(c, device, bytes, buf);
    if (st != GS_OK) return st;
    if (hipMemcpyAsync(buf.dev, host.data(), bytes, hipMemcpyHostToDevice, up) != hipSuccess ||
        hipStreamSynchronize(up) != hipSuccess) {
        c.retired.push_front(Retired{buf, {}});      // idle: reusable at once
        return GS_ERR_HIP;
    }
    cl.buf = buf;
    cl.nchunks = int64_t(host.size());
    return GS_OK;
}

// After a launch that reads the list on `stream`: pin the list when the
// stream is capturing (or its state cannot be read), else re-record the
// stream's event.
void note_use(CachedList &cl, hipStream_t stream) {
    if (cl.pinned) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        cl.pinned = true;
        return;
    }
    for (StreamUse &u : cl.uses)
        if (u.stream == stream) {
            if (hipEventRecord(u.event, stream) != hipSuccess) cl.pinned = true;
            return;
        }
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence) !=
        hipSuccess) {
        cl.pinned = true;
        return;
    }
    if (hipEventRecord(ev, stream) != hipSuccess) {
        (void)hipEventDestroy(ev);
        cl.pinned = true;
        return;
    }
    cl.uses.push_back(StreamUse{stream, ev});
}

// Evicts least recently used, unpinned lists until one more list of `need`
// bytes fits (or only pinned lists are left); their buffers are retired.
// Idle retired buffers beyond kCacheBytes on this device are moved to
// `to_free` (freed by the caller after the lock is released).
void make_room(ListCache &c, int device, size_t need, std::vector<void *> &to_free) {
    auto it = c.lru.end();
    while (it != c.lru.begin() && (c.map.size() >= kCacheEntries || c.bytes + need > kCacheBytes)) {
        --it;
        auto mit = c.map.find(*it);
        CachedList &old = mit->second.first;
        if (old.pinned) continue;
        c.bytes -= old.buf.cap;
        c.retired.push_front(Retired{old.buf, std::move(old.uses)});
        c.map.erase(mit);
        it = c.lru.erase(it);
    }
    size_t retired_bytes = 0;
    for (auto r = c.retired.begin(); r != c.retired.end();) {
        if (r->buf.device == device) {
            retired_bytes += r->buf.cap;
            if (retired_bytes > kCacheBytes && uses_done(r->uses)) {
                retired_bytes -= r->buf.cap;
                destroy_uses(r->uses);
                to_free.push_back(r->buf.dev);
                r = c.retired.erase(r);
                continue;
            }
        }
        ++r;
    }
}

// Looks up (or builds and caches) the list's descriptors and calls
// launch(list) with the cache lock held; then notes the launch's stream.
template <typename F>
gs_status with_list(int32_t n, const void *const *in, float *const *out, const int64_t *numel,
                    hipStream_t stream, F &&launch) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return GS_ERR_HIP;
    std::string key = make_key(device, n, in, out, numel);
    ListCache &c = cache();
    std::vector<void *> to_free;
    gs_status st;
    {
        std::lock_guard<std::mutex> lock(c.mu);
        auto it = c.map.find(key);
        if (it != c.map.end()) {
            c.lru.splice(c.lru.begin(), c.lru, it->second.second);
            CachedList &cl = it->second.first;
            st = launch(static_cast<const CachedList &>(cl));
            if (st == GS_OK) note_use(cl, stream);
            return st;
        }
        CachedList cl;
        st = build_list(c, device, n, in, out, numel, cl);
        if (st != GS_OK) return st;
        make_room(c, device, cl.buf.cap, to_free);
        c.lru.push_front(key);
        auto ins = c.map.emplace(key, std::make_pair(std::move(cl), c.lru.begin())).first;
        CachedList &added = ins->second.first;
        c.bytes += added.buf.cap;
        st = launch(static_cast<const CachedList &>(added));
        if (st == GS_OK) note_use(added, stream);
    }
    for (void *p : to_free) (void)hipFree(p);   // idle buffers past the retired limit
    return st;
}

inline bool bad_enum_fmt(int f) { return f != FP8_E4M3 && f != FP8_E5M2; }
inline bool bad_enum_gran(int g) {
    return g != FP8_PER_TENSOR && g != FP8_BLOCK_1x128 && g != FP8_BLOCK_128x128 &&
           g != FP8_BLOCK_1x32;
}

gs_status check_shape(int64_t rows, int64_t cols, int gran) {
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return GS_ERR_SIZE;
    if (rows * cols > kMaxElems) return GS_ERR_SIZE;
    if (gran == FP8_BLOCK_1x128 && cols % 128 != 0) return GS_ERR_SHAPE;
    if (gran == FP8_BLOCK_1x32 && cols % 32 != 0) return GS_ERR_SHAPE;
    if (gran == FP8_BLOCK_128x128 && (rows % 128 != 0 || cols % 128 != 0)) return GS_ERR_SHAPE;
    return GS_OK;
}

int64_t num_scales(int64_t rows, int64_t cols, int gran) {
    if (gran == FP8_PER_TENSOR) return 1;
    if (gran == FP8_BLOCK_1x128) return rows * (cols / 128);
    if (gran == FP8_BLOCK_1x32) return rows * (cols / 32);
    return (rows / 128) * (cols / 128);
}

inline bool misaligned(const void *p, uintptr_t a) { return (uintptr_t(p) & (a - 1)) != 0; }

inline gs_status from_hip(hipError_t e) { return e == hipSuccess ? GS_OK : GS_ERR_HIP; }

// Argument checks of a gradient list (pointers, counts, alignment); the
// element total in *total.
gs_status check_list(int32_t n, const void *const *grads, float *const *outs,
                     const int64_t *numels, int64_t *total) {
    *total = 0;
    if (n < 0) return GS_ERR_SIZE;
    if (n == 0) return GS_OK;
    if (!grads || !outs || !numels) return GS_ERR_NULL;
    for (int32_t i = 0; i < n; ++i) {
        if (numels[i] < 0 || numels[i] > kMaxElems) return GS_ERR_SIZE;
        if (numels[i] > 0 && (!grads[i] || !outs[i])) return GS_ERR_NULL;
        if (misaligned(grads[i], 2) || misaligned(outs[i], 4)) return GS_ERR_ALIGN;
        *total += numels[i];
        if (*total > kMaxElems * 64) return GS_ERR_SIZE;
    }
    return GS_OK;
}

}  // namespace

namespace gsk {

// Argument checks of an fp8_quantize call (everything but the workspace).
gs_status check_quantize(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                         fp8_format fmt, fp8_granularity g, fp8_scale_mode mode,
                         const uint8_t *codes, const float *scales, const int32_t *nonfinite) {
    if (x_dtype != GS_BF16 && x_dtype != GS_F32) return GS_ERR_DTYPE;
    if (bad_enum_fmt(fmt) || bad_enum_gran(g)) return GS_ERR_ARG;
    if (mode != FP8_SCALE_FROM_AMAX && mode != FP8_SCALE_GIVEN) return GS_ERR_ARG;
    const gs_status st = check_shape(rows, cols, g);
    if (st != GS_OK) return st;
    if (rows * cols > 0 && (!x || !codes)) return GS_ERR_NULL;
    if (num_scales(rows, cols, g) > 0 && !scales) return GS_ERR_NULL;
    if (misaligned(x, 16) || misaligned(codes, 16) || misaligned(scales, 4) ||
        misaligned(nonfinite, 4))
        return GS_ERR_ALIGN;
    return GS_OK;
}

}  // namespace gsk

extern "C" {

gs_status gs_unscale_check(int32_t n, const void *const *grads, float *const *outs,
                           const int64_t *numels, gs_dtype in_dtype, const float *scale,
                           int32_t *found_inf, void *stream) {
    if (n < 0) return GS_ERR_SIZE;
    if (in_dtype != GS_F16) return GS_ERR_DTYPE;
    if (!scale || !found_inf) return GS_ERR_NULL;
    if (misaligned(scale, 4) || misaligned(found_inf, 4)) return GS_ERR_ALIGN;
    int64_t total = 0;
    const gs_status vs = check_list(n, grads, outs, numels, &total);
    if (vs != GS_OK) return vs;
    if (total == 0) return GS_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return with_list(n, grads, outs, numels, s, [&](const CachedList &cl) {
        return from_hip(gsk::launch_unscale_check(static_cast<const gsk::ChunkDesc *>(cl.buf.dev),
                                                  cl.nchunks, scale, found_inf, s));
    });
}

int64_t gs_unscale_list_descriptors(int32_t n, const void *const *grads, float *const *outs,
                                    const int64_t *numels, uint64_t *desc_out, int64_t capacity) {
    int64_t total = 0;
    gs_status st = check_list(n, grads, outs, numels, &total);
    if (st != GS_OK) return st;
    std::vector<gsk::ChunkDesc> host;
    st = make_descriptors(n, grads, outs, numels, host);
    if (st != GS_OK) return st;
    const int64_t count = int64_t(host.size());
    if (desc_out) {
        if (capacity < count) return GS_ERR_SIZE;
        for (int64_t k = 0; k < count; ++k) {
            desc_out[2 * k] = host[size_t(k)].in_bits;
            desc_out[2 * k + 1] = host[size_t(k)].out_bits;
        }
    }
    return count;
}

size_t gs_unscale_check_sumsq_workspace_size(int32_t n, const int64_t *numels) {
    if (n < 0 || (n > 0 && !numels)) return 0;
    int64_t chunks = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (numels[i] < 0 || numels[i] > kMaxElems) return 0;
        chunks += (numels[i] + gsk::kUnscaleChunk - 1) / gsk::kUnscaleChunk;
    }
    return size_t(chunks + gsk::kSumsqL2) * gsk::kSumsqPartBytes;
}

gs_status gs_unscale_check_sumsq(int32_t n, const void *const *grads, float *const *outs,
                                 const int64_t *numels, gs_dtype in_dtype, const float *scale,
                                 int32_t *found_inf, uint64_t *sumsq, double *norm_sq,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    if (n < 0) return GS_ERR_SIZE;
    if (in_dtype != GS_F16) return GS_ERR_DTYPE;
    if (!scale || !found_inf || !sumsq || !norm_sq) return GS_ERR_NULL;
    if (misaligned(scale, 4) || misaligned(found_inf, 4) || misaligned(sumsq, 8) ||
        misaligned(norm_sq, 8))
        return GS_ERR_ALIGN;
    int64_t total = 0;
    const gs_status vs = check_list(n, grads, outs, numels, &total);
    if (vs != GS_OK) return vs;
    if (!workspace || workspace_bytes < gs_unscale_check_sumsq_workspace_size(n, numels))
        return GS_ERR_WORKSPACE;
    if (misaligned(workspace, 16)) return GS_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto launch = [&](const CachedList &cl) {
        return from_hip(gsk::launch_unscale_check_sumsq(
            static_cast<const gsk::ChunkDesc *>(cl.buf.dev), cl.nchunks, scale, found_inf, sumsq,
            norm_sq, workspace, s));
    };
    if (total == 0) return launch(CachedList{});   // still folds the total into norm_sq
    return with_list(n, grads, outs, numels, s, launch);
}

gs_status gs_update_scale(float *scale, int32_t *growth_tracker, int32_t *found_inf,
                          float growth_factor, float backoff_factor, int32_t growth_interval,
                          int64_t *skip_count, void *stream) {
    if (!scale || !growth_tracker || !found_inf) return GS_ERR_NULL;
    if (misaligned(scale, 4) || misaligned(growth_tracker, 4) || misaligned(found_inf, 4) ||
        misaligned(skip_count, 8))
        return GS_ERR_ALIGN;
    if (!(std::isfinite(growth_factor) && growth_factor > 0.0f)) return GS_ERR_ARG;
    if (!(std::isfinite(backoff_factor) && backoff_factor > 0.0f)) return GS_ERR_ARG;
    if (growth_interval <= 0) return GS_ERR_ARG;
    return from_hip(gsk::launch_update_scale(scale, growth_tracker, found_inf, growth_factor,
                                             backoff_factor, growth_interval, skip_count,
                                             static_cast<hipStream_t>(stream)));
}

gs_status gs_update_scale_hysteresis(float *scale, int32_t *growth_tracker,
                                     int32_t *hysteresis_left, int32_t *found_inf,
                                     float growth_factor, float backoff_factor,
                                     int32_t growth_interval, int32_t hysteresis,
                                     int32_t consecutive_hysteresis, float min_scale,
                                     int64_t *skip_count, void *stream) {
    if (!scale || !growth_tracker || !hysteresis_left || !found_inf) return GS_ERR_NULL;
    if (misaligned(scale, 4) || misaligned(growth_tracker, 4) || misaligned(hysteresis_left, 4) ||
        misaligned(found_inf, 4) || misaligned(skip_count, 8))
        return GS_ERR_ALIGN;
    if (!(std::isfinite(growth_factor) && growth_factor > 0.0f)) return GS_ERR_ARG;
    if (!(std::isfinite(backoff_factor) && backoff_factor > 0.0f)) return GS_ERR_ARG;
    if (growth_interval <= 0 || hysteresis < 1) return GS_ERR_ARG;
    if (consecutive_hysteresis != 0 && consecutive_hysteresis != 1) return GS_ERR_ARG;
    if (!(std::isfinite(min_scale) && min_scale >= 0.0f)) return GS_ERR_ARG;
    return from_hip(gsk::launch_update_scale_hysteresis(
        scale, growth_tracker, hysteresis_left, found_inf, growth_factor, backoff_factor,
        growth_interval, hysteresis, consecutive_hysteresis, min_scale, skip_count,
        static_cast<hipStream_t>(stream)));
}

size_t fp8_quantize_workspace_size(int64_t rows, int64_t cols, fp8_granularity g) {
    (void)rows;
    (void)cols;
    return g == FP8_PER_TENSOR ? size_t(gsk::kPartialSlots) * sizeof(uint32_t) : 0;
}

gs_status fp8_quantize(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                       fp8_format fmt, fp8_granularity g, fp8_scale_mode mode, uint8_t *codes,
                       float *scales, int32_t *nonfinite, void *workspace,
                       size_t workspace_bytes, void *stream) {
    const gs_status st = gsk::check_quantize(x, x_dtype, rows, cols, fmt, g, mode, codes,
                                             scales, nonfinite);
    if (st != GS_OK) return st;
    const bool need_ws = (g == FP8_PER_TENSOR && mode == FP8_SCALE_FROM_AMAX);
    if (need_ws) {
        if (!workspace || workspace_bytes < fp8_quantize_workspace_size(rows, cols, g))
            return GS_ERR_WORKSPACE;
        if (misaligned(workspace, 4)) return GS_ERR_ALIGN;
    }
    return from_hip(gsk::launch_quantize(x, x_dtype, rows, cols, fmt, g, mode, codes, scales,
                                         nonfinite, static_cast<uint32_t *>(workspace),
                                         static_cast<hipStream_t>(stream)));
}

gs_status fp8_quantize_delayed(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                               fp8_format fmt, float *scale_state, float *amax_history,
                               int32_t history_len, int32_t *history_pos, uint8_t *codes,
                               float *scale_used, int32_t *nonfinite, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (x_dtype != GS_BF16 && x_dtype != GS_F32) return GS_ERR_DTYPE;
    if (bad_enum_fmt(fmt)) return GS_ERR_ARG;
    if (history_len < 1 || history_len > gsk::kMaxHistory) return GS_ERR_ARG;
    gs_status st = check_shape(rows, cols, FP8_PER_TENSOR);
    if (st != GS_OK) return st;
    const int64_t n = rows * cols;
    if (n > 0 && (!x || !codes)) return GS_ERR_NULL;
    if (!scale_state || !amax_history || !history_pos || !scale_used) return GS_ERR_NULL;
    if (misaligned(x, 16) || misaligned(codes, 16) || misaligned(scale_state, 4) ||
        misaligned(amax_history, 4) || misaligned(history_pos, 4) || misaligned(scale_used, 4) ||
        misaligned(nonfinite, 4))
        return GS_ERR_ALIGN;
    if (!workspace || workspace_bytes < fp8_quantize_workspace_size(rows, cols, FP8_PER_TENSOR))
        return GS_ERR_WORKSPACE;
    if (misaligned(workspace, 4)) return GS_ERR_ALIGN;
    return from_hip(gsk::launch_quantize_delayed(
        x, x_dtype, rows, cols, fmt, scale_state, amax_history, history_len, history_pos, codes,
        scale_used, nonfinite, static_cast<uint32_t *>(workspace),
        static_cast<hipStream_t>(stream)));
}

gs_status fp8_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                         fp8_granularity g, const float *scales, float *out, void *stream) {
    if (bad_enum_fmt(fmt) || bad_enum_gran(g)) return GS_ERR_ARG;
    gs_status st = check_shape(rows, cols, g);
    if (st != GS_OK) return st;
    const int64_t n = rows * cols;
    if (n > 0 && (!codes || !out || !scales)) return GS_ERR_NULL;
    if (misaligned(codes, 16) || misaligned(out, 16) || misaligned(scales, 4)) return GS_ERR_ALIGN;
    if (n == 0) return GS_OK;
    return from_hip(gsk::launch_dequantize(codes, rows, cols, fmt, g, scales, out,
                                           static_cast<hipStream_t>(stream)));
}

gs_status fp8_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                              fp8_granularity g, const float *scales, uint16_t *out,
                              void *stream) {
    if (bad_enum_fmt(fmt) || bad_enum_gran(g)) return GS_ERR_ARG;
    gs_status st = check_shape(rows, cols, g);
    if (st != GS_OK) return st;
    const int64_t n = rows * cols;
    if (n > 0 && (!codes || !out || !scales)) return GS_ERR_NULL;
    if (misaligned(codes, 16) || misaligned(out, 16) || misaligned(scales, 4)) return GS_ERR_ALIGN;
    if (n == 0) return GS_OK;
    return from_hip(gsk::launch_dequantize_bf16(codes, rows, cols, fmt, g, scales, out,
                                                static_cast<hipStream_t>(stream)));
}

gs_status fp8_quantize_mx(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                          fp8_format fmt, uint8_t *codes, uint8_t *scales_e8m0,
                          int32_t *nonfinite, void *stream) {
    if (x_dtype != GS_BF16 && x_dtype != GS_F32) return GS_ERR_DTYPE;
    if (bad_enum_fmt(fmt)) return GS_ERR_ARG;
    const gs_status st = check_shape(rows, cols, FP8_BLOCK_1x32);
    if (st != GS_OK) return st;
    if (rows * cols > 0 && (!x || !codes || !scales_e8m0)) return GS_ERR_NULL;
    if (misaligned(x, 16) || misaligned(codes, 16) || misaligned(nonfinite, 4)) return GS_ERR_ALIGN;
    if (rows * cols == 0) return GS_OK;
    return from_hip(gsk::launch_quantize_mx(x, x_dtype, rows, cols, fmt, codes, scales_e8m0,
                                            nonfinite, static_cast<hipStream_t>(stream)));
}

gs_status fp8_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, fp8_format fmt,
                            const uint8_t *scales_e8m0, float *out, void *stream) {
    if (bad_enum_fmt(fmt)) return GS_ERR_ARG;
    const gs_status st = check_shape(rows, cols, FP8_BLOCK_1x32);
    if (st != GS_OK) return st;
    if (rows * cols > 0 && (!codes || !out || !scales_e8m0)) return GS_ERR_NULL;
    if (misaligned(codes, 16) || misaligned(out, 16)) return GS_ERR_ALIGN;
    if (rows * cols == 0) return GS_OK;
    return from_hip(gsk::launch_dequantize_mx(codes, rows, cols, fmt, scales_e8m0, out,
                                              static_cast<hipStream_t>(stream)));
}

const char *gs_status_string(gs_status status) {
    switch (status) {
        case GS_OK: return "GS_OK";
        case GS_ERR_NULL: return "GS_ERR_NULL: a required pointer is NULL";
        case GS_ERR_SIZE: return "GS_ERR_SIZE: negative or too large count or size";
        case GS_ERR_SHAPE: return "GS_ERR_SHAPE: block granularity does not divide the shape";
        case GS_ERR_DTYPE: return "GS_ERR_DTYPE: unsupported element type";
        case GS_ERR_ARG: return "GS_ERR_ARG: bad enum, factor or interval";
        case GS_ERR_ALIGN: return "GS_ERR_ALIGN: misaligned pointer";
        case GS_ERR_WORKSPACE: return "GS_ERR_WORKSPACE: workspace missing or too small";
        case GS_ERR_HIP: return "GS_ERR_HIP: HIP runtime or launch failure";
        default: return "unknown gs_status";
    }
}

}  // extern "C"
