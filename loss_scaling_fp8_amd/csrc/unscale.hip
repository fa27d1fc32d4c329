// unscale.hip -- fused multi-tensor FP16 -> FP32 unscale with a device-side
// non-finite check, and the grow/backoff loss-scale update.
//
// "Loss scaling, FP8, and the failure that never crashes", section "Loss
// scaling, derived from the chain rule you already have": backward produced
// S*g; the recovered gradient is g_scaled / S, formed in FP32; an Inf or NaN
// means S was too large, so the step is skipped and S halved; after a run of
// clean steps S is doubled.  The SimpleGradScaler listing of the worked
// example gives the control logic, "Numerical Precision, Mixed Precision, and
// Loss Scaling" the default factors (x2.0 / x0.5 / 2000).
//
// Design (gfx950): one launch covers the whole gradient list.  The list is
// cut into 2048-element chunks, each with a 16-byte descriptor (its input and
// output addresses, a ragged count, an alignment flag) built once on the
// host and cached on the device.  The grid is one 256-lane workgroup per
// chunk (grid-stride past 2^22 workgroups): a workgroup does one scalar load
// of its descriptor, then every lane moves 8 FP16 values as two 8-byte loads
// and two 16-byte non-temporal stores, so each wave-wide store instruction
// writes 1 KiB of contiguous FP32.  On MI355X this 1:2 read:write stream ran
// at the speed of the same kernel with no lookup at all, ahead of binary
// searches over the list, per-chunk tensor indices, persistent workgroups,
// and 32-byte-per-lane store layouts.  The finiteness test rides along in
// registers; a lane that saw a non-finite value stores 1 to the flag (plain
// vector store, idempotent).  The update is one lane of one wave; nothing
// ever comes back to the host.
#include "gs_internal.hpp"

#ifndef GS_UNSCALE_GRID_CAP
#define GS_UNSCALE_GRID_CAP (1 << 22)
#endif

namespace gsk {

namespace {

__device__ __forceinline__ float widen_f16(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h16);
}

// y = fl32(g * inv); canonical NaN on output; accumulate "not finite".
__device__ __forceinline__ float unscale_one(uint32_t h16, float inv, bool &bad) {
    const float y = widen_f16(h16) * inv;
    bad |= !__builtin_isfinite(y);
    return __builtin_isnan(y) ? __uint_as_float(0x7FC00000u) : y;
}

// The data addresses come from memory, so the compiler cannot tell that they
// are global; these types let it emit global (not flat) loads and stores.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x2 g_cu32x2;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
typedef __attribute__((address_space(1))) const uint16_t g_cu16;
typedef __attribute__((address_space(1))) float g_f32;

__global__ __launch_bounds__(kUnscaleThreads)
void unscale_check_kernel(const ChunkDesc *__restrict__ descs, int64_t nchunks,
                          const float *__restrict__ scale, int32_t *__restrict__ found_inf) {
    const float inv = 1.0f / *scale;         // IEEE division, once per lane
    bool bad = false;
    const int tid = threadIdx.x;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const ChunkDesc d = descs[c];
        g_cu16 *in = (g_cu16 *)(uintptr_t)(d.in_bits & kAddrMask);
        g_f32 *out = (g_f32 *)(uintptr_t)(d.out_bits & ~uint64_t(3));
        const int64_t ragged = int64_t(d.in_bits >> 48);
        if (ragged == 0 && (d.out_bits & 1) == 0) {
            g_cu32x2 *src = (g_cu32x2 *)in;
            g_f32x4 *dst = (g_f32x4 *)out;
            u32x2 v[kUnscaleUnroll];
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) v[u] = src[u * kUnscaleThreads + tid];
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) {
                const f32x4 y = {unscale_one(v[u].x & 0xFFFFu, inv, bad),
                                 unscale_one(v[u].x >> 16, inv, bad),
                                 unscale_one(v[u].y & 0xFFFFu, inv, bad),
                                 unscale_one(v[u].y >> 16, inv, bad)};
                __builtin_nontemporal_store(y, &dst[u * kUnscaleThreads + tid]);
            }
        } else {
            const int64_t cnt = ragged ? ragged : kUnscaleChunk;
            for (int64_t i = tid; i < cnt; i += kUnscaleThreads) out[i] = unscale_one(in[i], inv, bad);
        }
    }
    if (bad) *found_inf = 1;                 // idempotent; only ever 1
}

__global__ void update_scale_kernel(float *scale, int32_t *tracker, int32_t *found_inf,
                                    float growth, float backoff, int32_t interval,
                                    int64_t *skips) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    float S = *scale;
    if (*found_inf) {
        S = S * backoff;
        *tracker = 0;
        if (skips) *skips = *skips + 1;
    } else {
        int32_t t = *tracker + 1;
        if (t >= interval) {
            S = S * growth;
            t = 0;
        }
        *tracker = t;
    }
    *scale = S;
    *found_inf = 0;
}

}  // namespace

hipError_t launch_unscale_check(const ChunkDesc *descs, int64_t nchunks, const float *scale,
                                int32_t *found_inf, hipStream_t stream) {
    if (nchunks <= 0) return hipSuccess;
    const int64_t cap = GS_UNSCALE_GRID_CAP;
    const int64_t grid = nchunks < cap ? nchunks : cap;
    hipLaunchKernelGGL(unscale_check_kernel, dim3((uint32_t)grid), dim3(kUnscaleThreads), 0,
                       stream, descs, nchunks, scale, found_inf);
    return hipGetLastError();
}

hipError_t launch_update_scale(float *scale, int32_t *tracker, int32_t *found_inf, float growth,
                               float backoff, int32_t interval, int64_t *skips,
                               hipStream_t stream) {
    hipLaunchKernelGGL(update_scale_kernel, dim3(1), dim3(64), 0, stream, scale, tracker,
                       found_inf, growth, backoff, interval, skips);
    return hipGetLastError();
}

}  // namespace gsk
