// gs_internal.hpp -- declarations shared by the HIP translation units of
// libgsfp8 (not part of the public ABI; the public ABI is include/gs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gs.h"

namespace gsk {

// ---------------------------------------------------------------- unscale
// Device view of a cached multi-tensor work list.  Every tensor is cut into
// chunks of kUnscaleChunk elements (the last one ragged); chunk_begin is the
// prefix sum of the chunk counts, so a flat chunk id maps to its tensor by a
// binary search over n+1 entries.
struct WorkList {
    const int64_t *chunk_begin;   // [n + 1]
    const uint16_t *const *in;    // [n] FP16 gradients
    float *const *out;            // [n] FP32 outputs
    const int64_t *numel;         // [n]
    const int32_t *vec_ok;        // [n] 1 when both bases are 16-byte aligned
    int32_t n;
    int64_t total_chunks;
};

constexpr int kUnscaleThreads = 256;
constexpr int kUnscaleVec = 8;        // FP16 elements per 16-byte load
constexpr int kUnscaleUnroll = 4;     // loads in flight per lane per chunk
constexpr int64_t kUnscaleChunk = int64_t(kUnscaleThreads) * kUnscaleVec * kUnscaleUnroll;

hipError_t launch_unscale_check(const WorkList &wl, const float *scale, int32_t *found_inf,
                                hipStream_t stream);
hipError_t launch_update_scale(float *scale, int32_t *tracker, int32_t *found_inf, float growth,
                               float backoff, int32_t interval, int64_t *skips,
                               hipStream_t stream);

// ---------------------------------------------------------------- FP8
constexpr int kPartialSlots = 1024;   // per-tensor amax partials (workspace words)

hipError_t launch_quantize(const void *x, gs_dtype dt, int64_t rows, int64_t cols, int fmt,
                           int gran, int mode, uint8_t *codes, float *scales,
                           int32_t *nonfinite, uint32_t *partials, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, int fmt, int gran,
                             const float *scales, float *out, hipStream_t stream);

}  // namespace gsk
