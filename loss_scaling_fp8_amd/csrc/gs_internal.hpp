// gs_internal.hpp -- declarations shared by the HIP translation units of
// libgsfp8 (not part of the public ABI; the public ABI is include/gs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gs.h"

namespace gsk {

// ---------------------------------------------------------------- stores
// A 16-byte store with a chosen cache policy.  POLICY < 0 is an ordinary
// global store (-1 non-temporal, -2 plain); POLICY >= 0 is the policy field
// of a buffer store (gfx950: sc0 = 1, nt = 2, sc1 = 16), through a buffer
// resource at the wave-uniform address `base`; `off` is the lane's byte
// offset from `base`, any size for the global stores, below 2^31 for the
// buffer store (the resource's range is 2^31 - 1 bytes).
constexpr int kPolicyGlobalNt = -1;
constexpr int kPolicyGlobalPlain = -2;
typedef uint32_t st_u32x4 __attribute__((ext_vector_type(4)));

template <int POLICY, typename V>
__device__ __forceinline__ void store16(void *base, int64_t off, V v) {
    static_assert(sizeof(V) == 16, "16-byte stores only");
    const st_u32x4 w = __builtin_bit_cast(st_u32x4, v);
    if constexpr (POLICY == kPolicyGlobalNt) {
        __builtin_nontemporal_store(w, reinterpret_cast<st_u32x4 *>(static_cast<char *>(base) + off));
    } else if constexpr (POLICY == kPolicyGlobalPlain) {
        *reinterpret_cast<st_u32x4 *>(static_cast<char *>(base) + off) = w;
    } else {
        // raw (stride 0) resource; its last word sets the data-format field to
        // 32 bits (4 << 15), which gfx9-family buffer accesses need non-zero
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7FFFFFFF, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, POLICY);
    }
}

// ---------------------------------------------------------------- unscale
// The gradient list is cut into chunks of kUnscaleChunk elements (the last
// chunk of a tensor ragged), and each chunk gets a 16-byte descriptor built
// once on the host and cached on the device:
//   in_bits  = address of the chunk's first FP16 element (bits 0..47)
//              | element count << 48 when the chunk is ragged (else 0)
//   out_bits = address of the chunk's first FP32 output
//              | 1 when the tensor is not 16-byte aligned (element-wise path)
// One workgroup per chunk needs a single dependent (scalar) load before it
// streams its data.
struct ChunkDesc {
    uint64_t in_bits;
    uint64_t out_bits;
};

constexpr int kUnscaleThreads = 256;
constexpr int kUnscaleVec = 4;        // FP16 elements per 8-byte load (one 16-byte store)
constexpr int kUnscaleUnroll = 2;     // loads per lane per chunk
constexpr int64_t kUnscaleChunk = int64_t(kUnscaleThreads) * kUnscaleVec * kUnscaleUnroll;
constexpr uint64_t kAddrMask = (uint64_t(1) << 48) - 1;

hipError_t launch_unscale_check(const ChunkDesc *descs, int64_t nchunks, const float *scale,
                                int32_t *found_inf, hipStream_t stream);
// Unscale + exact gradient sum of squares: one 16-byte partial per chunk
// (workspace), then kSumsqL2 second-level 128-bit partials, then one
// workgroup adds them to the running total and writes the norm squared.
constexpr int kSumsqL2 = 1024;
constexpr size_t kSumsqPartBytes = 16;
hipError_t launch_unscale_check_sumsq(const ChunkDesc *descs, int64_t nchunks, const float *scale,
                                      int32_t *found_inf, uint64_t *sumsq, double *norm_sq,
                                      void *workspace, hipStream_t stream);
hipError_t launch_update_scale_hysteresis(float *scale, int32_t *tracker, int32_t *hleft,
                                          int32_t *found_inf, float growth, float backoff,
                                          int32_t window, int32_t hysteresis, int32_t consecutive,
                                          float min_scale, int64_t *skips, hipStream_t stream);
hipError_t launch_update_scale(float *scale, int32_t *tracker, int32_t *found_inf, float growth,
                               float backoff, int32_t interval, int64_t *skips,
                               hipStream_t stream);

// ---------------------------------------------------------------- FP8
constexpr int kPartialSlots = 8192;   // per-tensor amax partials (workspace words)

// Argument checks of an fp8_quantize call, everything but the workspace
// (defined in api.hip).
gs_status check_quantize(const void *x, gs_dtype x_dtype, int64_t rows, int64_t cols,
                         fp8_format fmt, fp8_granularity g, fp8_scale_mode mode,
                         const uint8_t *codes, const float *scales, const int32_t *nonfinite);

hipError_t launch_quantize(const void *x, gs_dtype dt, int64_t rows, int64_t cols, int fmt,
                           int gran, int mode, uint8_t *codes, float *scales,
                           int32_t *nonfinite, uint32_t *partials, hipStream_t stream);
constexpr int kMaxHistory = 1024;     // delayed scaling: amax history entries
hipError_t launch_quantize_delayed(const void *x, gs_dtype dt, int64_t rows, int64_t cols,
                                   int fmt, float *scale_state, float *history, int32_t hlen,
                                   int32_t *pos, uint8_t *codes, float *scale_used,
                                   int32_t *nonfinite, uint32_t *partials, hipStream_t stream);
hipError_t launch_quantize_mx(const void *x, gs_dtype dt, int64_t rows, int64_t cols, int fmt,
                              uint8_t *codes, uint8_t *scales, int32_t *nonfinite,
                              hipStream_t stream);
hipError_t launch_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                                const uint8_t *scales, float *out, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, int fmt, int gran,
                             const float *scales, float *out, hipStream_t stream);
hipError_t launch_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                                  int gran, const float *scales, uint16_t *out,
                                  hipStream_t stream);

}  // namespace gsk
