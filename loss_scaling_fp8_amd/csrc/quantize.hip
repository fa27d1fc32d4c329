// quantize.hip -- FP8 (OCP E4M3 / E5M2) scaled quantization at per-tensor,
// 1x128, 128x128 and 1x32 granularity (1x32 also with MX-style E8M0
// scales), and the matching dequantization.
//
// What is computed ("Mixed precision and FP8 training", section "FP8
// training", fp8_scaling.py: quant / per_tensor / per_block; "Why FP8
// training is stable", Failure 1 and "The seam"): per block, the largest
// finite |x| gives s = fl32(max(amax, 1e-12) / MAX); each element becomes
// the FP8 code of clamp(fl32(x / s), -MAX, MAX) rounded to nearest-even; the
// dequantized value is decode(code) * s in FP32.  The 1x32 blocks are the
// granularity of the MX formats (same page, hardware notes: one scaling
// factor per 32 elements); their power-of-two E8M0 scale is the smallest
// power of two not below the block scale above.
//
// Design (gfx950, wave64):
//  * 1x128: a row-major matrix whose width is a multiple of 128 is a flat
//    sequence of 128-element blocks, so the kernel walks blocks linearly.
//    A lane owns 32 contiguous elements (4 x 16-byte loads of BF16), a quad
//    of lanes owns a block: the block amax is two DPP quad exchanges, and
//    each lane stores 32 codes (2 x 16 bytes).
//  * 1x32 (and MX-style 1x32 with E8M0 power-of-two scales): the 1x128
//    walk with one lane per block, so the amax needs no lane exchange.
//  * 128x128: one 256-lane workgroup per tile, the whole tile held in
//    registers (64 elements per lane); amax by DPP inside rows of 16 lanes,
//    two cross-row shuffles, and 4 LDS words across the waves.
//  * per-tensor: the scale depends on the whole tensor, so the tensor is
//    read twice: a pass writes one partial max per workgroup (<= 8192; no
//    atomics, no zero-initialised memory), then the cast pass streams the
//    tensor again.  For a tensor that fits in the infinity cache the amax
//    pass writes at most 1024 partials and every cast workgroup reduces
//    them itself; a larger one has one 1024-lane workgroup turn them into
//    the scale in between.  Both passes use the 1x128 lane layout (a lane
//    owns 32 contiguous elements).  Delayed scaling casts with the previous
//    scale and emits the partials in the same pass, then updates the
//    history in one workgroup.
//  * dequantize: a flat walk over groups of codes (4 per lane with FP32
//    output, 8 with BF16), each lane one 16-byte store, so every wave-wide
//    store writes 1 KiB of contiguous output; 128x128 finds each group's
//    tile from its position.
//  * Division: x / s is formed from r = fl32(1/s) and one FMA correction
//    (div_by_scale) whenever s is in the range where that reproduces the
//    IEEE quotient's FP8 code, else by IEEE division (only a given scale
//    can be outside that range).  Lanes holding a NaN or Inf keep the fast
//    path and then rewrite just those codes; amax ignores them.
//  * The max-abs is taken on bit patterns: for non-negative floats unsigned
//    integer order is numeric order, and BF16 halves are maxed pairwise.
#include "device_fp8.hpp"
#include <atomic>
#include <type_traits>
#include "gs_internal.hpp"

// Cache policy per kernel (1 = non-temporal), chosen by measurement.
#ifndef GS_Q1_NT_LOAD
#define GS_Q1_NT_LOAD 0
#endif
#ifndef GS_Q1_NT_STORE
#define GS_Q1_NT_STORE 0
#endif
#ifndef GS_Q128_NT_LOAD
#define GS_Q128_NT_LOAD 1
#endif
#ifndef GS_Q128_NT_STORE
#define GS_Q128_NT_STORE 0
#endif
#ifndef GS_QT_NT_LOAD
#define GS_QT_NT_LOAD 0
#endif
#ifndef GS_QT_NT_STORE
#define GS_QT_NT_STORE 0
#endif
#ifndef Q128_THREADS
#define Q128_THREADS 256
#endif
// per-tensor scaling of a cache-resident tensor: partial maxima of the amax
// pass, pieces in flight per lane there and its load policy, and pieces
// per lane of the cast (which reduces the partials once per workgroup)
#ifndef GS_PT_FOLD_PARTS
#define GS_PT_FOLD_PARTS 1024
#endif
#ifndef GS_PT_AMAX_U
#define GS_PT_AMAX_U 2
#endif
#ifndef GS_PT_AMAX_NT
#define GS_PT_AMAX_NT 0
#endif
#ifndef GS_PT_CAST_PIECES
#define GS_PT_CAST_PIECES 2
#endif
// block quantizers: workgroups per CU (0 = as many as registers allow),
// capped by reserving LDS the kernels do not use; measured best: 6 for the
// row-block kernel (1x128, 1x32, MX), 5 for 128x128
// FP32-output dequantizers: groups of 4 codes per lane per work item (the
// linear walk; the 128x128 walk), and workgroups per CU (0 = no cap)
#ifndef GS_DQ_UNROLL_F32
#define GS_DQ_UNROLL_F32 2
#endif
#ifndef GS_DQT_UNROLL_F32
#define GS_DQT_UNROLL_F32 4
#endif
#ifndef GS_DQ_WGS_PER_CU
#define GS_DQ_WGS_PER_CU 0
#endif
#ifndef GS_Q1_WGS_PER_CU
#define GS_Q1_WGS_PER_CU 6
#endif
#ifndef GS_Q128_WGS_PER_CU
#define GS_Q128_WGS_PER_CU 5
#endif

namespace gsk {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void *p) {
    const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}

template <bool NT, typename V>
__device__ __forceinline__ void st(void *p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
    else *reinterpret_cast<V *>(p) = v;
}

constexpr uint32_t kFloorBits = 0x2B8CBCCCu;  // fl32(1e-12)

template <int FMT>
__device__ __forceinline__ float scale_from_amax(float amax) {
    const float fl = as_f32(kFloorBits);
    const float a = amax > fl ? amax : fl;
    return a / Fp8<FMT>::kMax;
}

// ---------------------------------------------------------------- lane data
// NV 16-byte vectors of input per lane, as 32-bit words.
template <typename IN, int NV>
struct LaneData {
    static constexpr int kPerVec = 16 / int(sizeof(IN));   // elements per vector
    static constexpr int kElems = NV * kPerVec;
    static constexpr int kWords = NV * 4;
    uint32_t w[kWords];

    template <bool NT>
    __device__ __forceinline__ void load(const IN *p) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32x4 t = ld16<NT>(p + i * kPerVec);
            w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
        }
    }
    // load NV vectors spaced `stride` elements apart
    template <bool NT>
    __device__ __forceinline__ void load_strided(const IN *p, int64_t stride) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32x4 t = ld16<NT>(p + i * stride);
            w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
        }
    }

    // FP32 bit pattern of element i (BF16 widened by appending 16 zeros)
    __device__ __forceinline__ uint32_t elem(int i) const {
        if constexpr (sizeof(IN) == 2)
            return (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
        else
            return w[i];
    }

    // Largest finite |x| of the lane as FP32 bits; returns true when the lane
    // holds a NaN or an Inf (those are left out of the max).
    __device__ __forceinline__ bool absmax(uint32_t &amax_bits) const {
        if constexpr (sizeof(IN) == 2) {
            typedef unsigned short us2 __attribute__((ext_vector_type(2)));
            us2 m = {0, 0};
#pragma unroll
            for (int i = 0; i < kWords; ++i)
                m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu));
            uint32_t m16 = m.x > m.y ? m.x : m.y;
            const bool nf = m16 >= 0x7F80u;
            if (nf) {
                m16 = 0;
#pragma unroll
                for (int i = 0; i < kWords; ++i) {
                    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
                    if (lo < 0x7F80u && lo > m16) m16 = lo;
                    if (hi < 0x7F80u && hi > m16) m16 = hi;
                }
            }
            amax_bits = m16 << 16;
            return nf;
        } else {
            // the maximum of the bits shifted left by one (the sign dropped,
            // the order kept): written unlike the fallback's |x| below, so
            // that the compiler does not keep every |x| alive for it
            uint32_t m2 = 0;
#pragma unroll
            for (int i = 0; i < kWords; ++i) m2 = max(m2, w[i] << 1);
            const bool nf = m2 >= (0x7F800000u << 1);
            uint32_t m = m2 >> 1;
            if (nf) {
                m = 0;
#pragma unroll
                for (int i = 0; i < kWords; ++i) {
                    const uint32_t a = w[i] & 0x7FFFFFFFu;
                    if (a < 0x7F800000u && a > m) m = a;
                }
            }
            amax_bits = m;
            return nf;
        }
    }

    // FP8 codes of all lane elements, 4 per output word (little-endian).
    // Fast path (scale in the fast range): |x| / s by the reciprocal and one
    // FMA correction, the sign of x put back, and the hardware conversion; a
    // clamp only when the scale was given (with a scale from this block's
    // amax, |x / s| <= MAX (1 + 2^-23) for every finite x).  A lane holding
    // a NaN or an Inf then rewrites just those codes: NaN -> sign|0x7F,
    // +-Inf -> +-MAX (Inf / s is infinite for a finite positive s, and the
    // clamp saturates it).  Other scales (0, negative, non-finite, tiny or
    // huge) take the IEEE division per element; they can only be given, so
    // that path is compiled only when GIVEN (a scale from a block amax is
    // always in the fast range, and leaving the path out frees registers).
    // The fix-up runs per group of 4 right after that group's codes, so its
    // inputs are live anyway: done as one pass after the whole lane, it kept
    // every unpacked element alive and cost 34 VGPRs (128x128: 130 -> 68
    // together with the fast-only amax path, 3 -> 7 workgroups per CU).
    template <int FMT, bool GIVEN>
    __device__ __forceinline__ void cast(float s, bool lane_nonfinite,
                                         uint32_t (&out)[kElems / 4]) const {
        const float r = 1.0f / s;
        if (!GIVEN || fast_scale(s)) {
            constexpr uint32_t kMaxCode = FMT == 0 ? 0x7Eu : 0x7Bu;
#pragma unroll
            for (int j = 0; j < kElems / 4; ++j) {
                float q[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t e = elem(4 * j + k);
                    float a = div_by_scale(__builtin_fabsf(as_f32(e)), s, r);
                    if (GIVEN) a = as_f32(min(as_u32(a), Fp8<FMT>::kMaxBits));
                    q[k] = as_f32(as_u32(a) | (e & 0x80000000u));
                }
                uint32_t o = cvt_pk<FMT, true>(q[2], q[3], cvt_pk<FMT, false>(q[0], q[1], 0u));
                if (lane_nonfinite) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t e = elem(4 * j + k);
                        if ((e & 0x7F800000u) == 0x7F800000u) {
                            const uint32_t c = ((e >> 24) & 0x80u) | ((e & 0x7FFFFFu) ? 0x7Fu : kMaxCode);
                            o = (o & ~(0xFFu << (8 * k))) | (c << (8 * k));
                        }
                    }
                }
                out[j] = o;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kElems / 4; ++j) {
                uint32_t acc = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc |= cast_exact<FMT>(as_f32(elem(4 * j + k)), s) << (8 * k);
                out[j] = acc;
            }
        }
    }
};

template <bool NT>
__device__ __forceinline__ void store_words(uint8_t *p, const uint32_t *w, int nwords) {
    // nwords is a compile-time multiple of 1..4 words; 16-byte pieces first
    int i = 0;
    for (; i + 4 <= nwords; i += 4) st<NT>(p + 4 * i, u32x4{w[i], w[i + 1], w[i + 2], w[i + 3]});
    for (; i + 2 <= nwords; i += 2) st<NT>(p + 4 * i, u32x2{w[i], w[i + 1]});
    for (; i < nwords; ++i) st<NT>(p + 4 * i, w[i]);
}

// ---------------------------------------------------------------- 1x128, 1x32
// A lane owns 32 contiguous elements (BF16: 4 vectors, FP32: 8), so a
// 1x128 block is a quad of lanes (amax by DPP quad exchanges) and a 1x32
// block is one lane; either way lane l of a wave reads bytes [64 l, 64 l +
// 64) of the wave's span (BF16), the same access pattern.
// MODE: FP8_SCALE_FROM_AMAX and FP8_SCALE_GIVEN (FP32 scales), or kModeMx:
// the amax scale rounded up to a power of two, written as its E8M0 byte
// (the FP32 exponent field: both biases are 127).
constexpr int kModeMx = 2;

template <int FMT, int MODE, typename IN, int BLOCK>
__global__ __launch_bounds__(256)
void quant_row_blocks_kernel(const IN *__restrict__ x, int64_t nblocks,
                             uint8_t *__restrict__ codes, void *__restrict__ scales,
                             int32_t *__restrict__ nonfinite) {
    constexpr int kElems = 32;
    constexpr int kLanesPerBlock = BLOCK / kElems;           // 4 or 1
    constexpr int NV = kElems * int(sizeof(IN)) / 16;
    constexpr int kBlocksPerWG = 256 / kLanesPerBlock;
    const int sub = threadIdx.x & (kLanesPerBlock - 1);
    bool saw_nf = false;
    for (int64_t b = int64_t(blockIdx.x) * kBlocksPerWG + (threadIdx.x / kLanesPerBlock);
         b < nblocks; b += int64_t(gridDim.x) * kBlocksPerWG) {
        LaneData<IN, NV> L;
        L.template load<GS_Q1_NT_LOAD>(x + b * BLOCK + sub * kElems);
        uint32_t amax_bits;
        const bool nf = L.absmax(amax_bits);
        saw_nf |= nf;
        float s;
        if (MODE == FP8_SCALE_GIVEN) {
            s = static_cast<const float *>(scales)[b];
        } else {
            amax_bits = group_max<kLanesPerBlock>(amax_bits);
            s = scale_from_amax<FMT>(as_f32(amax_bits));
            if (MODE == kModeMx) {
                uint32_t sb = as_u32(s);                      // positive, normal, < 2^120
                if (sb & 0x7FFFFFu) sb = (sb & 0x7F800000u) + 0x00800000u;
                s = as_f32(sb);
                if (sub == 0) static_cast<uint8_t *>(scales)[b] = (uint8_t)(sb >> 23);
            } else if (sub == 0) {
                static_cast<float *>(scales)[b] = s;
            }
        }
        uint32_t out[kElems / 4];
        L.template cast<FMT, MODE == FP8_SCALE_GIVEN>(s, nf, out);
        store_words<GS_Q1_NT_STORE>(codes + b * BLOCK + sub * kElems, out, kElems / 4);
    }
    if (saw_nf && nonfinite) *nonfinite = 1;
}

// ---------------------------------------------------------------- 128x128
// One workgroup of T lanes per tile.  Threads per 128-element row: 16 (BF16)
// or 32 (FP32), one 16-byte vector each; the tile takes 128 / (T / threads
// per row) row passes.
template <int FMT, int MODE, typename IN, int T = Q128_THREADS>
__global__ __launch_bounds__(T)
void quant_128x128_kernel(const IN *__restrict__ x, int64_t cols, int64_t tiles_per_row,
                          int64_t ntiles, uint8_t *__restrict__ codes, float *__restrict__ scales,
                          int32_t *__restrict__ nonfinite) {
    constexpr int kPerVec = 16 / int(sizeof(IN));
    constexpr int kThreadsPerRow = 128 / kPerVec;
    constexpr int kRowsPerPass = T / kThreadsPerRow;
    constexpr int kPasses = 128 / kRowsPerPass;
    constexpr int kWaves = T / 64;
    __shared__ uint32_t red[kWaves];
    const int tid = threadIdx.x;
    const int row0 = tid / kThreadsPerRow;
    const int seg = tid % kThreadsPerRow;
    bool saw_nf = false;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t ti = t / tiles_per_row, tj = t - ti * tiles_per_row;
        const int64_t base = (ti * 128 + row0) * cols + tj * 128 + seg * kPerVec;
        // the row stride, opaque per tile: keeps the compiler from hoisting
        // one 64-bit address per pass out of the tile loop (32 VGPRs with
        // FP32 input)
        int64_t rs = int64_t(kRowsPerPass) * cols;
        __asm__ volatile("" : "+s"(rs));
        LaneData<IN, kPasses> L;
        L.template load_strided<GS_Q128_NT_LOAD>(x + base, rs);
        uint32_t amax_bits;
        const bool nf = L.absmax(amax_bits);
        saw_nf |= nf;
        float s;
        if (MODE == FP8_SCALE_FROM_AMAX) {
            amax_bits = wave_max(amax_bits);
            if ((tid & 63) == 0) red[tid >> 6] = amax_bits;
            __syncthreads();
            amax_bits = red[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) amax_bits = max(amax_bits, red[w]);
            __syncthreads();                  // red[] is reused by the next tile
            s = scale_from_amax<FMT>(as_f32(amax_bits));
            if (tid == 0) scales[t] = s;
        } else {
            s = scales[t];
        }
        uint32_t out[LaneData<IN, kPasses>::kElems / 4];
        L.template cast<FMT, MODE == FP8_SCALE_GIVEN>(s, nf, out);
        // each pass contributes kPerVec codes of one row
        constexpr int kWordsPerPass = kPerVec / 4;
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            uint8_t *dst = codes + base + int64_t(p) * rs;
            if constexpr (kWordsPerPass == 2)
                st<GS_Q128_NT_STORE>(dst, u32x2{out[2 * p], out[2 * p + 1]});
            else
                st<GS_Q128_NT_STORE>(dst, out[p]);
        }
    }
    if (saw_nf && nonfinite) *nonfinite = 1;
}

// ---------------------------------------------------------------- per-tensor
// Pass 1: one partial finite max (FP32 bits) per workgroup (<= 8192
// workgroups, grid-stride).  Two layouts, chosen by the tensor's size:
//  * the tensor fits in the 256 MB infinity cache (STREAM = false): the lane
//    layout of the cast below, a lane reading a piece of 32 contiguous
//    elements with plain loads, so the cast's second read hits the cache;
//  * larger tensors (STREAM = true): units of 4 x 256 consecutive 16-byte
//    vectors (each wave-wide load reads 1 KiB of contiguous input) with
//    non-temporal loads.
// Measured on MI355X: 8192x8192 BF16 61.4 -> 59.1 us with the first for the
// whole quantize, four 16384x32768 BF16 tensors 3.70 -> 3.49 TB/s with it,
// hence the switch.  Workgroup 0 takes the elements past the last whole
// piece / vector.
constexpr int64_t kCacheResidentBytes = int64_t(192) << 20;

template <typename IN, bool STREAM>
__global__ __launch_bounds__(256)
void amax_partials_kernel(const IN *__restrict__ x, int64_t n, uint32_t *__restrict__ partials,
                          int32_t *__restrict__ nonfinite) {
    constexpr int kStep = STREAM ? 16 / int(sizeof(IN)) : 32;   // elements per lane load unit
    __shared__ uint32_t red[4];
    const int64_t nunits = n / kStep;
    uint32_t m = 0;
    bool nf = false;
    if constexpr (STREAM) {
        constexpr int U = 4;
        for (int64_t v0 = int64_t(blockIdx.x) * 256 * U; v0 < nunits;
             v0 += int64_t(gridDim.x) * 256 * U) {
            LaneData<IN, 1> L[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = v0 + u * 256 + threadIdx.x;
                if (v < nunits) L[u].template load<true>(x + v * kStep);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t v = v0 + u * 256 + threadIdx.x;
                if (v < nunits) {
                    uint32_t a;
                    nf |= L[u].absmax(a);
                    m = max(m, a);
                }
            }
        }
    } else {
        constexpr int NV = kStep * int(sizeof(IN)) / 16;
        constexpr int U = GS_PT_AMAX_U;
        for (int64_t b0 = int64_t(blockIdx.x) * 256 * U + threadIdx.x; b0 < nunits;
             b0 += int64_t(gridDim.x) * 256 * U) {
            LaneData<IN, NV> L[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (b0 + u * 256 < nunits) L[u].template load<GS_PT_AMAX_NT>(x + (b0 + u * 256) * kStep);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (b0 + u * 256 < nunits) {
                    uint32_t a;
                    nf |= L[u].absmax(a);
                    m = max(m, a);
                }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nunits * kStep) {     // ragged tail
        const IN *p = x + nunits * kStep + threadIdx.x;
        uint32_t b;
        if constexpr (sizeof(IN) == 2) b = uint32_t(*reinterpret_cast<const uint16_t *>(p)) << 16;
        else b = *reinterpret_cast<const uint32_t *>(p);
        b &= 0x7FFFFFFFu;
        if (b >= 0x7F800000u) nf = true; else m = max(m, b);
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
    if (nf && nonfinite) *nonfinite = 1;
}

// Pass 2 (one 1024-lane workgroup): the tensor amax from the partials (all
// loads issued before any is used), and its scale.
template <int FMT>
__global__ __launch_bounds__(1024)
void amax_finalize_kernel(const uint32_t *__restrict__ partials, int nparts,
                          float *__restrict__ scales) {
    constexpr int kPer = kPartialSlots / 1024;
    __shared__ uint32_t red[16];
    uint32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = k * 1024 + threadIdx.x;
        v[k] = i < nparts ? partials[i] : 0u;
    }
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) m = max(m, v[k]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < 16; ++w) r = max(r, red[w]);
        scales[0] = scale_from_amax<FMT>(as_f32(r));
    }
}

// Pass 3 (the only pass with a given scale): cast with the scale in
// scales[0].  The lane layout of the 1x128 kernel: a lane owns a piece of
// 32 contiguous elements (BF16: 4 vectors; FP32: 8) and stores its 32 codes
// as two 16-byte words; pieces are walked grid-stride, and the fewer than
// 32 elements past the last whole piece are cast one per lane by workgroup
// 0.  (Walking single 16-byte vectors, each wave-wide load reading 1 KiB of
// contiguous input and storing 8 codes per lane, ran 22% slower on the
// 8192x8192 pair.)  With EMIT (delayed scaling), each workgroup also
// writes the largest finite |x| it saw to partials[blockIdx.x]; the grid
// then has <= kPartialSlots workgroups.
//
// With FOLD (a tensor of at most kCacheResidentBytes, whose amax pass then
// writes at most kFoldParts partials), pass 2 is folded in: every workgroup
// first reduces the partials itself (four 4-byte loads per lane, from L2)
// and derives the scale, and workgroup 0 writes it to scales[0].  That drops
// a launch: 8192x8192 BF16 ran 1.5-3% faster, a 1024x1024 tensor 12-20%.
// Streamed tensors keep pass 2: capping their amax pass at kFoldParts
// workgroups cost them 5%.  (Loading the first piece before the fold, to
// overlap the two, gained nothing; 2048 partials cost 6%.)
constexpr int kFoldParts = GS_PT_FOLD_PARTS;
static_assert(kFoldParts % 256 == 0 && kFoldParts <= kPartialSlots, "fold partials");

template <int FMT, bool GIVEN, typename IN, bool EMIT = false, bool FOLD = false>
__global__ __launch_bounds__(256)
void quant_tensor_kernel(const IN *__restrict__ x, int64_t n, uint8_t *__restrict__ codes,
                         float *scales, int32_t *__restrict__ nonfinite,
                         uint32_t *__restrict__ partials = nullptr, int nparts = 0) {
    constexpr int kElems = 32;
    constexpr int NV = kElems * int(sizeof(IN)) / 16;
    float s;
    if constexpr (FOLD) {
        __shared__ uint32_t pred[4];
        uint32_t pm = 0;
#pragma unroll
        for (int k = 0; k < kFoldParts / 256; ++k) {
            const int i = k * 256 + threadIdx.x;
            if (i < nparts) pm = max(pm, partials[i]);
        }
        pm = wave_max(pm);
        if ((threadIdx.x & 63) == 0) pred[threadIdx.x >> 6] = pm;
        __syncthreads();
        s = scale_from_amax<FMT>(as_f32(max(max(pred[0], pred[1]), max(pred[2], pred[3]))));
        if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = s;
    } else {
        s = scales[0];
    }
    bool saw_nf = false;
    uint32_t m = 0;
    const int64_t npieces = n / kElems;
    for (int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x; b < npieces;
         b += int64_t(gridDim.x) * 256) {
        LaneData<IN, NV> L;
        L.template load<GS_QT_NT_LOAD>(x + b * kElems);
        uint32_t a;
        const bool nf = L.absmax(a);
        saw_nf |= nf;
        m = max(m, a);
        uint32_t out[kElems / 4];
        L.template cast<FMT, GIVEN>(s, nf, out);
        store_words<GS_QT_NT_STORE>(codes + b * kElems, out, kElems / 4);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - npieces * kElems) {     // ragged tail
        const int64_t i = npieces * kElems + threadIdx.x;
        uint32_t bits;
        if constexpr (sizeof(IN) == 2) bits = uint32_t(reinterpret_cast<const uint16_t *>(x)[i]) << 16;
        else bits = reinterpret_cast<const uint32_t *>(x)[i];
        if ((bits & 0x7FFFFFFFu) >= 0x7F800000u) saw_nf = true;
        else m = max(m, bits & 0x7FFFFFFFu);
        codes[i] = (uint8_t)cast_exact<FMT>(as_f32(bits), s);
    }
    if (saw_nf && nonfinite) *nonfinite = 1;
    if constexpr (EMIT) {
        __shared__ uint32_t red[4];
        m = wave_max(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        if (threadIdx.x == 0) partials[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
    }
}

// Delayed scaling, history update (one 1024-lane workgroup): this step's
// amax from the partials into the ring, the next step's scale as the
// maximum over the window, the scale this step used.
template <int FMT>
__global__ __launch_bounds__(1024)
void delayed_update_kernel(const uint32_t *__restrict__ partials, int nparts,
                           float *__restrict__ scale_state, float *__restrict__ history,
                           int32_t hlen, int32_t *__restrict__ pos,
                           float *__restrict__ scale_used) {
    constexpr int kPer = kPartialSlots / 1024;
    __shared__ uint32_t red[16];
    __shared__ uint32_t amax_t;
    uint32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = k * 1024 + threadIdx.x;
        v[k] = i < nparts ? partials[i] : 0u;
    }
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) m = max(m, v[k]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < 16; ++w) r = max(r, red[w]);
        amax_t = r;
    }
    __syncthreads();
    // window maximum with this step's amax in slot p (history values are
    // non-negative floats, so their bit patterns order like their values)
    const int32_t p = ((*pos % hlen) + hlen) % hlen;
    const int32_t tid = int32_t(threadIdx.x);
    uint32_t h = 0;
    if (tid < hlen)
        h = (tid == p) ? amax_t : as_u32(history[tid]);
    h = wave_max(h);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = h;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t hm = 0;
        for (int w = 0; w < 16; ++w) hm = max(hm, red[w]);
        *scale_used = *scale_state;
        history[p] = as_f32(amax_t);
        *pos = (p + 1) % hlen;
        *scale_state = scale_from_amax<FMT>(as_f32(hm));
    }
}

// ---------------------------------------------------------------- dequantize
// A lane turns a group of codes into one 16-byte non-temporal store, so
// every wave-wide store instruction writes 1 KiB of contiguous output: 4
// codes (one 4-byte load) into 4 FP32 values, or 8 codes (one 8-byte load)
// into 8 BF16 values, rounded by gfx950's v_cvt_pk_bf16_f32 (round to
// nearest even; checked against that rounding on all 2^32 FP32 inputs).
// OUT: float or uint16_t (BF16 bits).
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename OUT>
struct DqGroup {
    static constexpr int kCodes = sizeof(OUT) == 4 ? 4 : 8;    // codes per lane per group
    // groups per lane per work item of the flat walk.  BF16: 2, measured
    // back to back 1.3% ahead of 4 on 16384x7168 codes.  FP32, linear walk:
    // 2, ahead of 4 by 7% cold and 10% on 16384x32768 codes (8 lost 6%);
    // FP32, 128x128 walk: 4 (2 was within +-2%).
    static constexpr int kUnroll = sizeof(OUT) == 4 ? GS_DQ_UNROLL_F32 : 2;
    static constexpr int kUnrollTiles = sizeof(OUT) == 4 ? GS_DQT_UNROLL_F32 : 2;
    typedef typename std::conditional<kCodes == 4, uint32_t, u32x2>::type Word;
};

// Two FP32 values rounded to BF16 (a in the low half): one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    const bf16x2_t h = __builtin_convertvector(f32x2{a, b}, bf16x2_t);
    uint32_t r;
    __builtin_memcpy(&r, &h, sizeof(r));
    return r;
}

template <int FMT>
__device__ __forceinline__ void dequant_group(uint32_t w, float s, float *dst) {
    float v[4];
    decode4<FMT>(w, v);
    const f32x4 o = {canon(v[0] * s), canon(v[1] * s), canon(v[2] * s), canon(v[3] * s)};
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4 *>(dst));
}

template <int FMT>
__device__ __forceinline__ void dequant_group(u32x2 w, float s, uint16_t *dst) {
    float v[8];
    decode4<FMT>(w.x, *reinterpret_cast<float(*)[4]>(v));
    decode4<FMT>(w.y, *reinterpret_cast<float(*)[4]>(v + 4));
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = canon(v[k] * s);
    __builtin_nontemporal_store(u32x4{bf16x2(v[0], v[1]), bf16x2(v[2], v[3]),
                                      bf16x2(v[4], v[5]), bf16x2(v[6], v[7])},
                                reinterpret_cast<u32x4 *>(dst));
}

template <int FMT>
__device__ __forceinline__ float dequant_one(uint8_t c, float s) {
    float v[4];
    decode4<FMT>(c, v);
    return canon(v[0] * s);
}

// Scale of a 1x32 block from its E8M0 byte: 2^(b - 127), NaN for 0xFF
// (b = 0 is the FP32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_scale(uint32_t b) {
    return b == 0xFFu ? as_f32(0x7FC00000u) : as_f32(b ? (b << 23) : 0x00400000u);
}

// Flat walk over groups of 4 codes (FP32 output) or 8 (BF16).  KIND: 0
// per-tensor, 1 1x128, 2 1x32 with FP32 scales, 3 1x32 with E8M0 scale
// bytes; a block holds a whole number of groups.
template <int FMT, int KIND, typename OUT>
__global__ __launch_bounds__(256)
void dequant_linear_kernel(const uint8_t *__restrict__ codes, int64_t n,
                           const void *__restrict__ scales_v, OUT *__restrict__ out) {
    constexpr int U = DqGroup<OUT>::kUnroll;
    constexpr bool BLOCKED = KIND != 0;
    constexpr int kCodes = DqGroup<OUT>::kCodes;
    constexpr int kShift = kCodes == 4 ? 2 : 3;                // log2(codes per group)
    typedef typename DqGroup<OUT>::Word Word;
    const float *scales = static_cast<const float *>(scales_v);
    const int64_t ngroups = n / kCodes;
    const float s0 = BLOCKED ? 0.0f : scales[0];
    const Word *cw = reinterpret_cast<const Word *>(codes);
    for (int64_t g0 = int64_t(blockIdx.x) * 256 * U; g0 < ngroups;
         g0 += int64_t(gridDim.x) * 256 * U) {
        Word w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u * 256 + threadIdx.x;
            w[u] = g < ngroups ? cw[g] : Word{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u * 256 + threadIdx.x;
            if (g < ngroups) {
                float s = s0;
                if (KIND == 1) s = scales[g >> (7 - kShift)];
                if (KIND == 2) s = scales[g >> (5 - kShift)];
                if (KIND == 3) s = e8m0_scale(static_cast<const uint8_t *>(scales_v)[g >> (5 - kShift)]);
                dequant_group<FMT>(w[u], s, out + g * kCodes);
            }
        }
    }
    if (!BLOCKED && blockIdx.x == 0 && threadIdx.x < n - ngroups * kCodes) {
        const int64_t i = ngroups * kCodes + threadIdx.x;
        const float v = dequant_one<FMT>(codes[i], s0);
        if constexpr (sizeof(OUT) == 4) out[i] = v;
        else out[i] = (OUT)(bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

// 128x128: the same flat walk over the codes in row-major order, so that
// every wave-wide store still writes 1 KiB of contiguous output (a walk over
// tiles writes 512-byte row pieces 4 x cols bytes apart, and ran 6-12% slower
// cold).  Each group finds its tile's scale from its row and 128-code column
// block: per work item, one division gives the row r0 and block cb0 of its
// first group; per group, the quotient of its block count by the blocks per
// row, nb, comes from the FP32 reciprocal of nb and is off by at most one
// (operands below 2^24), which one comparison each way fixes.  (A 32-bit
// index with a single comparison for rows of 32 or more blocks issues fewer
// instructions but ran 2% slower with FP32 output.)
template <int FMT, typename OUT>
__global__ __launch_bounds__(256)
void dequant_tiles_kernel(const uint8_t *__restrict__ codes, int64_t n, int64_t cols,
                          uint32_t nb, float inv_nb, const float *__restrict__ scales,
                          OUT *__restrict__ out) {
    constexpr int U = DqGroup<OUT>::kUnrollTiles;
    constexpr int kCodes = DqGroup<OUT>::kCodes;
    typedef typename DqGroup<OUT>::Word Word;
    const int64_t ngroups = n / kCodes;
    const Word *cw = reinterpret_cast<const Word *>(codes);
    for (int64_t g0 = int64_t(blockIdx.x) * 256 * U; g0 < ngroups;
         g0 += int64_t(gridDim.x) * 256 * U) {
        const int64_t i0 = g0 * kCodes;                        // a multiple of 128
        const int64_t r0 = i0 / cols;
        const uint32_t cb0 = uint32_t((i0 - r0 * cols) >> 7);
        Word w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u * 256 + threadIdx.x;
            w[u] = g < ngroups ? cw[g] : Word{};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + u * 256 + threadIdx.x;
            if (g < ngroups) {
                const uint32_t cb = cb0 + (uint32_t((u * 256 + threadIdx.x) * kCodes) >> 7);
                uint32_t q = uint32_t(float(cb) * inv_nb);
                int32_t rem = int32_t(cb - q * nb);
                if (rem < 0) {
                    --q;
                    rem += int32_t(nb);
                } else if (rem >= int32_t(nb)) {
                    ++q;
                    rem -= int32_t(nb);
                }
                const int64_t row = r0 + q;
                dequant_group<FMT>(w[u], scales[(row >> 7) * nb + rem], out + g * kCodes);
            }
        }
    }
}

// Largest grid of any launch here; past it the kernels stride.  A test build
// sets a tiny cap, so that every grid-stride path runs at small sizes.
#ifndef GS_MAX_GRID
#define GS_MAX_GRID (1 << 20)
#endif
constexpr int64_t kMaxGrid = GS_MAX_GRID;

// Dynamic LDS that caps a block quantizer at `wgs` workgroups per CU (0: no
// cap), from the device's LDS per CU (queried once per device).
inline unsigned quant_lds_reserve(int wgs) {
    if (wgs <= 0) return 0;
    static std::atomic<int> lds_per_cu[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int lds = lds_per_cu[dev].load(std::memory_order_relaxed);
    if (lds <= 0) {
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess || lds <= 0)
            return 0;
        lds_per_cu[dev].store(lds, std::memory_order_relaxed);
    }
    return unsigned(lds) / unsigned(wgs + 1) + 1024u;
}

inline uint32_t grid_for(int64_t work_items, int64_t per_wg) {
    int64_t g = (work_items + per_wg - 1) / per_wg;
    if (g < 1) g = 1;
    if (g > kMaxGrid) g = kMaxGrid;
    return (uint32_t)g;
}

template <int FMT, int MODE, typename IN, int BLOCK>
hipError_t quantize_rows(const IN *x, int64_t n, uint8_t *codes, void *scales,
                         int32_t *nonfinite, hipStream_t stream) {
    const int64_t nblocks = n / BLOCK;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL((quant_row_blocks_kernel<FMT, MODE, IN, BLOCK>),
                       dim3(grid_for(nblocks, 256 / (BLOCK / 32))), dim3(256),
                       quant_lds_reserve(GS_Q1_WGS_PER_CU), stream, x, nblocks, codes, scales,
                       nonfinite);
    return hipGetLastError();
}

template <int FMT, int MODE, typename IN>
hipError_t quantize_typed(const IN *x, int64_t rows, int64_t cols, int gran, uint8_t *codes,
                          float *scales, int32_t *nonfinite, uint32_t *partials,
                          hipStream_t stream) {
    const int64_t n = rows * cols;
    if (gran == FP8_BLOCK_1x128)
        return quantize_rows<FMT, MODE, IN, 128>(x, n, codes, scales, nonfinite, stream);
    if (gran == FP8_BLOCK_1x32)
        return quantize_rows<FMT, MODE, IN, 32>(x, n, codes, scales, nonfinite, stream);
    if (gran == FP8_BLOCK_128x128) {
        const int64_t tpr = cols / 128, ntiles = (rows / 128) * tpr;
        if (ntiles == 0) return hipSuccess;
        hipLaunchKernelGGL((quant_128x128_kernel<FMT, MODE, IN>), dim3(grid_for(ntiles, 1)),
                           dim3(Q128_THREADS), quant_lds_reserve(GS_Q128_WGS_PER_CU), stream, x,
                           cols, tpr, ntiles, codes, scales, nonfinite);
        return hipGetLastError();
    }
    // per-tensor: partial maxima, the scale, the cast (given mode: the cast);
    // a cache-resident tensor folds the scale into the cast
    if (MODE == FP8_SCALE_FROM_AMAX) {
        const bool stream_big = n * int64_t(sizeof(IN)) > kCacheResidentBytes;
        const int64_t unit = stream_big ? 16 / int64_t(sizeof(IN)) * 256 * 4 : 32 * 256;
        int64_t p = (n + unit - 1) / unit;
        if (p < 1) p = 1;
        if (p > (stream_big ? kPartialSlots : kFoldParts)) p = stream_big ? kPartialSlots : kFoldParts;
        if (p > kMaxGrid) p = kMaxGrid;
        if (stream_big)
            hipLaunchKernelGGL((amax_partials_kernel<IN, true>), dim3((uint32_t)p), dim3(256), 0,
                               stream, x, n, partials, nonfinite);
        else
            hipLaunchKernelGGL((amax_partials_kernel<IN, false>), dim3((uint32_t)p), dim3(256), 0,
                               stream, x, n, partials, nonfinite);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (!stream_big) {
            hipLaunchKernelGGL((quant_tensor_kernel<FMT, false, IN, false, true>),
                               dim3(grid_for(n / 32, 256 * GS_PT_CAST_PIECES)), dim3(256), 0,
                               stream, x, n, codes, scales, nonfinite, partials, (int)p);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((amax_finalize_kernel<FMT>), dim3(1), dim3(1024), 0, stream, partials,
                           (int)p, scales);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((quant_tensor_kernel<FMT, MODE == FP8_SCALE_GIVEN, IN>),
                       dim3(grid_for(n / 32, 256)), dim3(256), 0, stream, x, n, codes,
                       scales, nonfinite);
    return hipGetLastError();
}

template <int FMT, typename IN>
hipError_t quantize_delayed_typed(const IN *x, int64_t rows, int64_t cols, float *scale_state,
                                  float *history, int32_t hlen, int32_t *pos, uint8_t *codes,
                                  float *scale_used, int32_t *nonfinite, uint32_t *partials,
                                  hipStream_t stream) {
    const int64_t n = rows * cols;
    int64_t g = (n / 32 + 255) / 256;            // one 32-element piece per lane
    if (g < 1) g = 1;
    if (g > kPartialSlots) g = kPartialSlots;
    if (g > kMaxGrid) g = kMaxGrid;
    hipLaunchKernelGGL((quant_tensor_kernel<FMT, true, IN, true>), dim3((uint32_t)g), dim3(256),
                       0, stream, x, n, codes, scale_state, nonfinite, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((delayed_update_kernel<FMT>), dim3(1), dim3(1024), 0, stream, partials,
                       (int)g, scale_state, history, hlen, pos, scale_used);
    return hipGetLastError();
}

template <int FMT, typename OUT>
hipError_t dequantize_fmt(const uint8_t *codes, int64_t rows, int64_t cols, int gran,
                          const float *scales, OUT *out, hipStream_t stream) {
    const int64_t n = rows * cols;
    if (n == 0) return hipSuccess;
    const dim3 grid(grid_for(n / DqGroup<OUT>::kCodes, 256 * DqGroup<OUT>::kUnroll));
    const unsigned dq_lds = sizeof(OUT) == 4 ? quant_lds_reserve(GS_DQ_WGS_PER_CU) : 0u;
    if (gran == FP8_BLOCK_128x128) {
        const dim3 tgrid(grid_for(n / DqGroup<OUT>::kCodes, 256 * DqGroup<OUT>::kUnrollTiles));
        const uint32_t nb = uint32_t(cols / 128);              // <= 2^24
        hipLaunchKernelGGL((dequant_tiles_kernel<FMT, OUT>), tgrid, dim3(256), dq_lds, stream, codes, n,
                           cols, nb, 1.0f / float(nb), scales, out);
        return hipGetLastError();
    }
    if (gran == FP8_BLOCK_1x128)
        hipLaunchKernelGGL((dequant_linear_kernel<FMT, 1, OUT>), grid, dim3(256), dq_lds, stream, codes,
                           n, scales, out);
    else if (gran == FP8_BLOCK_1x32)
        hipLaunchKernelGGL((dequant_linear_kernel<FMT, 2, OUT>), grid, dim3(256), dq_lds, stream, codes,
                           n, scales, out);
    else
        hipLaunchKernelGGL((dequant_linear_kernel<FMT, 0, OUT>), grid, dim3(256), dq_lds, stream, codes,
                           n, scales, out);
    return hipGetLastError();
}

template <int FMT>
hipError_t dequantize_mx_fmt(const uint8_t *codes, int64_t n, const uint8_t *scales, float *out,
                             hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((dequant_linear_kernel<FMT, 3, float>),
                       dim3(grid_for(n / 4, 256 * DqGroup<float>::kUnroll)),
                       dim3(256), quant_lds_reserve(GS_DQ_WGS_PER_CU), stream, codes, n, scales,
                       out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *x, gs_dtype dt, int64_t rows, int64_t cols, int fmt,
                           int gran, int mode, uint8_t *codes, float *scales,
                           int32_t *nonfinite, uint32_t *partials, hipStream_t stream) {
#define GS_Q(F, M, T) \
    return quantize_typed<F, M, T>(static_cast<const T *>(x), rows, cols, gran, codes, scales, \
                                   nonfinite, partials, stream)
#define GS_Q_T(F, M) \
    if (dt == GS_BF16) GS_Q(F, M, uint16_t); else GS_Q(F, M, float)
    if (fmt == FP8_E4M3) {
        if (mode == FP8_SCALE_FROM_AMAX) { GS_Q_T(0, 0); } else { GS_Q_T(0, 1); }
    } else {
        if (mode == FP8_SCALE_FROM_AMAX) { GS_Q_T(1, 0); } else { GS_Q_T(1, 1); }
    }
#undef GS_Q_T
#undef GS_Q
}

hipError_t launch_quantize_delayed(const void *x, gs_dtype dt, int64_t rows, int64_t cols,
                                   int fmt, float *scale_state, float *history, int32_t hlen,
                                   int32_t *pos, uint8_t *codes, float *scale_used,
                                   int32_t *nonfinite, uint32_t *partials, hipStream_t stream) {
#define GS_QD(F, T)                                                                            \
    return quantize_delayed_typed<F, T>(static_cast<const T *>(x), rows, cols, scale_state,   \
                                        history, hlen, pos, codes, scale_used, nonfinite,     \
                                        partials, stream)
    if (fmt == FP8_E4M3) {
        if (dt == GS_BF16) GS_QD(0, uint16_t); else GS_QD(0, float);
    } else {
        if (dt == GS_BF16) GS_QD(1, uint16_t); else GS_QD(1, float);
    }
#undef GS_QD
}

hipError_t launch_quantize_mx(const void *x, gs_dtype dt, int64_t rows, int64_t cols, int fmt,
                              uint8_t *codes, uint8_t *scales, int32_t *nonfinite,
                              hipStream_t stream) {
    const int64_t n = rows * cols;
    if (fmt == FP8_E4M3) {
        if (dt == GS_BF16)
            return quantize_rows<0, kModeMx, uint16_t, 32>(static_cast<const uint16_t *>(x), n,
                                                           codes, scales, nonfinite, stream);
        return quantize_rows<0, kModeMx, float, 32>(static_cast<const float *>(x), n, codes,
                                                    scales, nonfinite, stream);
    }
    if (dt == GS_BF16)
        return quantize_rows<1, kModeMx, uint16_t, 32>(static_cast<const uint16_t *>(x), n, codes,
                                                       scales, nonfinite, stream);
    return quantize_rows<1, kModeMx, float, 32>(static_cast<const float *>(x), n, codes, scales,
                                                nonfinite, stream);
}

hipError_t launch_dequantize_mx(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                                const uint8_t *scales, float *out, hipStream_t stream) {
    if (fmt == FP8_E4M3) return dequantize_mx_fmt<0>(codes, rows * cols, scales, out, stream);
    return dequantize_mx_fmt<1>(codes, rows * cols, scales, out, stream);
}

hipError_t launch_dequantize(const uint8_t *codes, int64_t rows, int64_t cols, int fmt, int gran,
                             const float *scales, float *out, hipStream_t stream) {
    if (fmt == FP8_E4M3) return dequantize_fmt<0>(codes, rows, cols, gran, scales, out, stream);
    return dequantize_fmt<1>(codes, rows, cols, gran, scales, out, stream);
}

hipError_t launch_dequantize_bf16(const uint8_t *codes, int64_t rows, int64_t cols, int fmt,
                                  int gran, const float *scales, uint16_t *out,
                                  hipStream_t stream) {
    if (fmt == FP8_E4M3) return dequantize_fmt<0>(codes, rows, cols, gran, scales, out, stream);
    return dequantize_fmt<1>(codes, rows, cols, gran, scales, out, stream);
}

}  // namespace gsk
