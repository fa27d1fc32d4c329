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
// cut into 8192-element chunks; a workgroup takes chunks in a grid-stride
// loop, finds the chunk's tensor by binary search over the chunk prefix sums,
// and streams it with 16-byte loads (8 FP16) and 16-byte stores (4 FP32).
// The finiteness test rides along in registers; one plain vector store of 1
// per wave that saw a non-finite value raises the flag.  The update is one
// lane of one wave; nothing ever comes back to the host.
#include "device_fp8.hpp"
#include "gs_internal.hpp"

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

// The tensor pointers come from memory, so the compiler cannot tell that they
// address global memory; casting them lets it emit global (not flat) loads
// and stores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_cu32x4;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
typedef __attribute__((address_space(1))) const uint16_t g_cu16;
typedef __attribute__((address_space(1))) float g_f32;

__device__ __forceinline__ int find_tensor(const WorkList &wl, int64_t chunk) {
    int lo = 0, hi = wl.n - 1;               // largest t with chunk_begin[t] <= chunk
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (wl.chunk_begin[mid] <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kUnscaleThreads)
void unscale_check_kernel(WorkList wl, const float *__restrict__ scale,
                          int32_t *__restrict__ found_inf) {
    const float inv = 1.0f / *scale;         // IEEE division, once per lane
    bool bad = false;
    const int tid = threadIdx.x;
    for (int64_t c = blockIdx.x; c < wl.total_chunks; c += gridDim.x) {
        const int t = find_tensor(wl, c);
        g_cu16 *__restrict__ in = (g_cu16 *)wl.in[t];
        g_f32 *__restrict__ out = (g_f32 *)wl.out[t];
        const int64_t start = (c - wl.chunk_begin[t]) * kUnscaleChunk;
        const int64_t rem = wl.numel[t] - start;
        if (rem >= kUnscaleChunk && wl.vec_ok[t]) {
            g_cu32x4 *src = (g_cu32x4 *)(in + start);
            g_f32x4 *dst = (g_f32x4 *)(out + start);
            u32x4 v[kUnscaleUnroll];
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) v[u] = src[u * kUnscaleThreads + tid];
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                float y[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    y[2 * k] = unscale_one(w[k] & 0xFFFFu, inv, bad);
                    y[2 * k + 1] = unscale_one(w[k] >> 16, inv, bad);
                }
                const int64_t o = int64_t(u * kUnscaleThreads + tid) * 2;
                dst[o] = f32x4{y[0], y[1], y[2], y[3]};
                dst[o + 1] = f32x4{y[4], y[5], y[6], y[7]};
            }
        } else {
            const int64_t cnt = rem < kUnscaleChunk ? rem : kUnscaleChunk;
            for (int64_t i = tid; i < cnt; i += kUnscaleThreads)
                out[start + i] = unscale_one(in[start + i], inv, bad);
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

hipError_t launch_unscale_check(const WorkList &wl, const float *scale, int32_t *found_inf,
                                hipStream_t stream) {
    if (wl.total_chunks <= 0) return hipSuccess;
    // Enough workgroups to keep every CU streaming (256 CUs x 8 resident
    // 256-lane workgroups), grid-stride beyond that.
    const int64_t cap = 256 * 8 * 4;
    const int64_t grid = wl.total_chunks < cap ? wl.total_chunks : cap;
    hipLaunchKernelGGL(unscale_check_kernel, dim3((uint32_t)grid), dim3(kUnscaleThreads), 0,
                       stream, wl, scale, found_inf);
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
