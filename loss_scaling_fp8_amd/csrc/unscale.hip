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
// ever comes back to the host.  The launch reserves unused LDS to hold the
// kernel to 7 workgroups per CU, which measured faster than the 8 its
// registers allow.  The sum-of-squares pass is left at those 8: each of its
// workgroups also reduces its chunk's sums (two workgroup barriers), and on
// the Llama-3-8B set it ran 2.3% faster uncapped (7.31 against 7.48 ms).
#include "gs_internal.hpp"

#include <atomic>

// Store policy of the outputs (see store16): device-scope non-temporal
// (sc1 nt).  On the Llama-3-8B set, ten launches back to back ran 1.3%
// faster than with plain non-temporal stores, and the benchmark step (the
// 1x128 quantize runs next) 0.6% faster.  The dequantizers keep plain
// non-temporal stores: with sc1 their writes drain into the next kernel
// (back to back they ran 16-19% slower).
#ifndef GS_UNSCALE_STORE
#define GS_UNSCALE_STORE 18
#endif
#ifndef GS_UNSCALE_GRID_CAP
#define GS_UNSCALE_GRID_CAP (1 << 22)
#endif

namespace gsk {

namespace {

__device__ __forceinline__ float widen_f16(uint32_t h16) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h16);
}

// y = fl32(g * inv); canonical NaN on output; accumulate "not finite".
__device__ __forceinline__ float unscale_f(float g, float inv, bool &bad) {
    const float y = g * inv;
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

// ---- exact sum of squares (the SUMSQ variant)
// A finite FP16 g is a multiple of 2^-24 below 2^16, so q = g*g is exact in
// FP32 (22-bit significand, in [2^-48, 2^32]) and G^2 = q * 2^48 is an
// integer.  Each q is split exactly in FP64 at the 2^-18 grid: t = q + C
// with C = 1.5 * 2^34 (ulp 2^-18; t stays in [2^34, 2^35)), hi = t - C,
// lo = q - hi (|lo| <= 2^-19, a multiple of 2^-48).  Per lane, over the 8
// elements of a chunk, sum(lo) is exact in FP64 and sum(hi) is carried as
// the integer sum of bits(t) - bits(C) (= hi * 2^18 per element), so the
// chunk's sum of G^2 = B * 2^30 + A with B = sum(hi) * 2^18 < 2^61 and
// |A| = |sum(lo)| * 2^48 <= 2^40, both exact 64-bit integers.
constexpr double kSplitC = 0x1.8p34;
constexpr uint64_t kSplitBits = 0x4218000000000000ull;   // bits of 1.5 * 2^34
constexpr double kIntMagic = 0x1.8p52;                  // integer extraction, |v| < 2^51
constexpr uint64_t kIntMagicBits = 0x4338000000000000ull;

__device__ __forceinline__ void sq_add(float f, double &lo, uint64_t &hib) {
    const double d = (double)(f * f);
    const double t = d + kSplitC;
    const double hi = t - kSplitC;
    lo += d - hi;
    hib += (uint64_t)__double_as_longlong(t);
}

// Sum over each row of 16 lanes (every lane of the row gets the row's sum),
// by DPP lane exchanges on the two 32-bit halves; all 64 lanes active.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t row_sum_u64(uint64_t v) {
    v += dpp_u64<0xB1>(v);     // quad_perm 1,0,3,2
    v += dpp_u64<0x4E>(v);     // quad_perm 2,3,0,1
    v += dpp_u64<0x141>(v);    // row_half_mirror: the other quad of each 8
    v += dpp_u64<0x140>(v);    // row_mirror: the other 8 of the row
    return v;
}

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

template <bool SUMSQ>
__global__ __launch_bounds__(kUnscaleThreads)
void unscale_check_kernel(const ChunkDesc *__restrict__ descs, int64_t nchunks,
                          const float *__restrict__ scale, int32_t *__restrict__ found_inf,
                          u64x2 *__restrict__ parts) {
    const float inv = 1.0f / *scale;         // IEEE division, once per lane
    bool bad = false;
    const int tid = threadIdx.x;
    __shared__ uint64_t red[2][kUnscaleThreads / 16];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const ChunkDesc d = descs[c];
        g_cu16 *in = (g_cu16 *)(uintptr_t)(d.in_bits & kAddrMask);
        g_f32 *out = (g_f32 *)(uintptr_t)(d.out_bits & ~uint64_t(3));
        const int64_t ragged = int64_t(d.in_bits >> 48);
        double lo = 0.0;                     // SUMSQ: this lane's sum of lo parts
        uint64_t hib = 0;                    // SUMSQ: sum of bits(t) - bits(C)
        if (ragged == 0 && (d.out_bits & 1) == 0) {
            g_cu32x2 *src = (g_cu32x2 *)in;
            u32x2 v[kUnscaleUnroll];
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) v[u] = src[u * kUnscaleThreads + tid];
            if (SUMSQ) hib = uint64_t(0) - uint64_t(kUnscaleUnroll * kUnscaleVec) * kSplitBits;
#pragma unroll
            for (int u = 0; u < kUnscaleUnroll; ++u) {
                const float f0 = widen_f16(v[u].x & 0xFFFFu), f1 = widen_f16(v[u].x >> 16);
                const float f2 = widen_f16(v[u].y & 0xFFFFu), f3 = widen_f16(v[u].y >> 16);
                const f32x4 y = {unscale_f(f0, inv, bad), unscale_f(f1, inv, bad),
                                 unscale_f(f2, inv, bad), unscale_f(f3, inv, bad)};
                store16<GS_UNSCALE_STORE>((void *)(uintptr_t)(d.out_bits & ~uint64_t(3)),
                                          uint32_t(u * kUnscaleThreads + tid) * 16u, y);
                if (SUMSQ) {
                    sq_add(f0, lo, hib);
                    sq_add(f1, lo, hib);
                    sq_add(f2, lo, hib);
                    sq_add(f3, lo, hib);
                }
            }
            // A non-finite input makes lo NaN; redo this lane's share with
            // Inf and NaN replaced by 0 (which adds t = C, i.e. hi = lo = 0).
            if (SUMSQ && !__builtin_isfinite(lo)) {
                lo = 0.0;
                hib = uint64_t(0) - uint64_t(kUnscaleUnroll * kUnscaleVec) * kSplitBits;
#pragma unroll
                for (int u = 0; u < kUnscaleUnroll; ++u) {
                    const uint32_t w[2] = {v[u].x, v[u].y};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float f = widen_f16((w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu);
                        sq_add(__builtin_isfinite(f) ? f : 0.0f, lo, hib);
                    }
                }
            }
        } else {
            const int64_t cnt = ragged ? ragged : kUnscaleChunk;
            for (int64_t i = tid; i < cnt; i += kUnscaleThreads) {
                const float f = widen_f16(in[i]);
                out[i] = unscale_f(f, inv, bad);
                if (SUMSQ && __builtin_isfinite(f)) {
                    sq_add(f, lo, hib);
                    hib -= kSplitBits;
                }
            }
        }
        if (SUMSQ) {
            // lo * 2^48 is an integer of magnitude <= 2^32: read it off the
            // bits of lo * 2^48 + 1.5 * 2^52 (exact).
            const double m = lo * 0x1p48 + kIntMagic;
            uint64_t a = (uint64_t)__double_as_longlong(m) - kIntMagicBits;
            uint64_t b = hib;
            a = row_sum_u64(a);
            b = row_sum_u64(b);
            if ((tid & 15) == 0) {
                red[0][tid >> 4] = b;
                red[1][tid >> 4] = a;
            }
            __syncthreads();
            if (tid == 0) {
                uint64_t sb = 0, sa = 0;
#pragma unroll
                for (int w = 0; w < kUnscaleThreads / 16; ++w) {
                    sb += red[0][w];
                    sa += red[1][w];
                }
                parts[c] = u64x2{sb, sa};     // chunk sum = sb * 2^30 + (int64)sa
            }
            __syncthreads();
        }
    }
    if (bad) *found_inf = 1;                 // idempotent; only ever 1
}

// 128-bit running sums as (lo, hi) word pairs
__device__ __forceinline__ void add128(uint64_t &lo, uint64_t &hi, uint64_t blo, uint64_t bhi) {
    lo += blo;
    hi += bhi + (lo < blo ? 1u : 0u);
}

// Sum of the 128-bit values (lo[i], hi[i]) of a workgroup's threads; the
// result is valid in thread 0.
template <int T>
__device__ __forceinline__ void block_sum128(uint64_t &lo, uint64_t &hi) {
    __shared__ uint64_t slo[T], shi[T];
    const int tid = threadIdx.x;
    slo[tid] = lo;
    shi[tid] = hi;
    __syncthreads();
#pragma unroll
    for (int s = T / 2; s > 0; s >>= 1) {
        if (tid < s) {
            uint64_t l = slo[tid], h = shi[tid];
            add128(l, h, slo[tid + s], shi[tid + s]);
            slo[tid] = l;
            shi[tid] = h;
        }
        __syncthreads();
    }
    lo = slo[0];
    hi = shi[0];
}

constexpr int kSumsqThreads = 256;

// Second level: each workgroup adds a strided share of the chunk partials
// (X = B * 2^30 + A, A signed) into one 128-bit value.
__global__ __launch_bounds__(kSumsqThreads)
void sumsq_reduce_kernel(const u64x2 *__restrict__ parts, int64_t nparts,
                         u64x2 *__restrict__ level2) {
    uint64_t lo = 0, hi = 0;
    for (int64_t i = int64_t(blockIdx.x) * kSumsqThreads + threadIdx.x; i < nparts;
         i += int64_t(gridDim.x) * kSumsqThreads) {
        const u64x2 p = parts[i];
        add128(lo, hi, p.x << 30, p.x >> 34);
        add128(lo, hi, p.y, (int64_t)p.y < 0 ? ~uint64_t(0) : uint64_t(0));
    }
    block_sum128<kSumsqThreads>(lo, hi);
    if (threadIdx.x == 0) level2[blockIdx.x] = u64x2{lo, hi};
}

// Round-to-nearest-even conversion of the 128-bit integer hi * 2^64 + lo.
__device__ double u128_to_f64(uint64_t hi, uint64_t lo) {
    uint64_t m, sticky;
    int sh;                                  // value = (m + f) * 2^sh, 0 <= f < 1, sticky = f != 0
    if (hi == 0) {
        m = lo;
        sticky = 0;
        sh = 0;
    } else {
        const int hb = 64 - __clzll((long long)hi);    // 1..64
        if (hb == 64) {
            m = hi;
            sticky = lo != 0;
        } else {
            m = (hi << (64 - hb)) | (lo >> hb);
            sticky = (lo << (64 - hb)) != 0;
        }
        sh = hb;
    }
    if (m < (uint64_t(1) << 53)) return ldexp((double)m, sh);   // exact (sticky is 0 here)
    const int drop = 11 - __clzll((long long)m);                  // keep 53 bits
    uint64_t keep = m >> drop;
    const uint64_t rem = m & ((uint64_t(1) << drop) - 1);
    const uint64_t half = uint64_t(1) << (drop - 1);
    if (rem > half || (rem == half && (sticky || (keep & 1)))) keep += 1;
    return ldexp((double)keep, sh + drop);                        // keep <= 2^53: exact
}

// Final: add the second-level values to the running total sumsq[0] +
// sumsq[1] * 2^64 and write norm_sq = (fl64(total) * 2^-48) * (inv * inv).
__global__ __launch_bounds__(kSumsqThreads)
void sumsq_final_kernel(const u64x2 *__restrict__ level2, int32_t n2,
                        const float *__restrict__ scale, uint64_t *__restrict__ sumsq,
                        double *__restrict__ norm_sq) {
    uint64_t lo = 0, hi = 0;
    for (int i = threadIdx.x; i < n2; i += kSumsqThreads) add128(lo, hi, level2[i].x, level2[i].y);
    block_sum128<kSumsqThreads>(lo, hi);
    if (threadIdx.x == 0) {
        add128(lo, hi, sumsq[0], sumsq[1]);
        sumsq[0] = lo;
        sumsq[1] = hi;
        const float inv = 1.0f / *scale;
        const double i2 = (double)inv * (double)inv;             // exact
        *norm_sq = (u128_to_f64(hi, lo) * 0x1p-48) * i2;
    }
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

// The same update with a hysteresis budget h, a floor on S and a growth
// window: an overflow restarts the window and either lowers S (budget spent:
// S = max(fl32(S * backoff), min_scale)) or spends one unit of budget; a
// clean step refills the budget when `consecutive`, and a growth refills it
// otherwise.
__global__ void update_scale_hysteresis_kernel(float *scale, int32_t *tracker, int32_t *hleft,
                                               int32_t *found_inf, float growth, float backoff,
                                               int32_t window, int32_t H, int32_t consecutive,
                                               float min_scale, int64_t *skips) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    float S = *scale;
    int32_t t = *tracker, h = *hleft;
    if (*found_inf) {
        if (skips) *skips = *skips + 1;
        t = 0;
        if (h <= 1) {
            const float lowered = S * backoff;
            S = lowered > min_scale ? lowered : min_scale;
        } else {
            h -= 1;
        }
    } else {
        if (consecutive) h = H;
        t += 1;
        if (t >= window) {
            S = S * growth;
            t = 0;
            if (!consecutive) h = H;
        }
    }
    *scale = S;
    *tracker = t;
    *hleft = h;
    *found_inf = 0;
}

// Occupancy cap for the unscale stream: LDS that the kernel does not use is
// reserved so that at most 7 of its workgroups share a CU (reservation =
// LDS per CU / 8 + 1 KiB).  At the 8 per CU its registers allow, MI355X
// ran the Llama-3-8B gradient set 6-7% slower (7.7-7.9 ms against 7.28 ms):
// more requests in flight than the memory system serves best.  Queried once
// per device.  The sum-of-squares pass does not use it (see the top of the
// file).
constexpr int kMaxDevices = 64;
std::atomic<unsigned> g_lds_reserve[kMaxDevices];

unsigned unscale_lds_reserve() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    unsigned r = g_lds_reserve[dev].load(std::memory_order_relaxed);
    if (r == 0) {
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess || lds <= 0)
            return 0;
        r = unsigned(lds) / 8 + 1024;
        g_lds_reserve[dev].store(r, std::memory_order_relaxed);
    }
    return r;
}

}  // namespace

hipError_t launch_update_scale_hysteresis(float *scale, int32_t *tracker, int32_t *hleft,
                                          int32_t *found_inf, float growth, float backoff,
                                          int32_t window, int32_t hysteresis, int32_t consecutive,
                                          float min_scale, int64_t *skips, hipStream_t stream) {
    hipLaunchKernelGGL(update_scale_hysteresis_kernel, dim3(1), dim3(64), 0, stream, scale,
                       tracker, hleft, found_inf, growth, backoff, window, hysteresis,
                       consecutive, min_scale, skips);
    return hipGetLastError();
}

hipError_t launch_unscale_check(const ChunkDesc *descs, int64_t nchunks, const float *scale,
                                int32_t *found_inf, hipStream_t stream) {
    if (nchunks <= 0) return hipSuccess;
    const int64_t cap = GS_UNSCALE_GRID_CAP;
    const int64_t grid = nchunks < cap ? nchunks : cap;
    hipLaunchKernelGGL(unscale_check_kernel<false>, dim3((uint32_t)grid), dim3(kUnscaleThreads),
                       unscale_lds_reserve(), stream, descs, nchunks, scale, found_inf,
                       (u64x2 *)nullptr);
    return hipGetLastError();
}

hipError_t launch_unscale_check_sumsq(const ChunkDesc *descs, int64_t nchunks, const float *scale,
                                      int32_t *found_inf, uint64_t *sumsq, double *norm_sq,
                                      void *workspace, hipStream_t stream) {
    u64x2 *parts = static_cast<u64x2 *>(workspace);
    u64x2 *level2 = parts + nchunks;
    int32_t n2 = 0;
    if (nchunks > 0) {
        const int64_t cap = GS_UNSCALE_GRID_CAP;
        const int64_t grid = nchunks < cap ? nchunks : cap;
        hipLaunchKernelGGL(unscale_check_kernel<true>, dim3((uint32_t)grid),
                           dim3(kUnscaleThreads), 0, stream, descs, nchunks, scale, found_inf,
                           parts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // about 8 or more partials per second-level thread
        const int64_t want = (nchunks + 8 * kSumsqThreads - 1) / (8 * kSumsqThreads);
        n2 = int32_t(want < kSumsqL2 ? want : kSumsqL2);
        hipLaunchKernelGGL(sumsq_reduce_kernel, dim3((uint32_t)n2), dim3(kSumsqThreads), 0,
                           stream, parts, nchunks, level2);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sumsq_final_kernel, dim3(1), dim3(kSumsqThreads), 0, stream, level2, n2,
                       scale, sumsq, norm_sq);
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
