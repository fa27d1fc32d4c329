// stream_ceilings.hip -- streaming kernels that measure the achievable HBM
// rate of each access pattern the library's kernels use, on flat buffers of
// the same sizes.  They do the least work a pattern allows and exist only
// for measurement: the benchmark times every variant below and reports each
// library kernel's rate as a fraction of the best rate of its pattern.
//
// Patterns (n = elements; a lane handles U units per chunk of 256 * U
// units: unit u * 256 + lane (layout 0: every wave-wide access is
// contiguous) or lane * U + u (layout 1: each lane's U units are
// contiguous, the layout of the quantizers' lanes)):
//   0 read only        16-byte loads, XOR-folded (n = bytes / 16 units)
//   1 write only       16-byte stores             (n = bytes / 16 units)
//   2 2 B -> 4 B       4 FP16 -> 4 FP32 per unit (8-byte load, 16-byte store):
//                      the unscale's pattern
//   3 2 B -> 1 B       16 BF16 -> 16 bytes per unit (two 16-byte loads, one
//                      16-byte store; the high byte of each value): the
//                      quantizers' pattern
//   4 1 B -> 4 B       4 bytes -> 4 FP32 per unit (4-byte load, 16-byte
//                      store): the FP32 dequantizers' pattern
//   5 1 B -> 2 B       8 bytes -> 8 16-bit values per unit (8-byte load,
//                      16-byte store): the BF16 dequantizers' pattern
// Variants: U in {1, 2, 4, 8}; layout 0 or 1; plain or non-temporal loads; store policy 0
// plain, 1 non-temporal, 2 a buffer store with the device-scope
// non-temporal policy (sc1 nt); and an occupancy cap of k workgroups per CU
// (0 = none), made by reserving LDS the kernel does not use.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int64_t kMaxGrid = int64_t(1) << 22;

template <bool NT, typename V>
__device__ __forceinline__ V get(const V *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int POLICY>
__device__ __forceinline__ void put16(void *chunk_base, uint32_t off, u32x4 v) {
    if constexpr (POLICY == 0) {
        *reinterpret_cast<u32x4 *>(static_cast<char *>(chunk_base) + off) = v;
    } else if constexpr (POLICY == 1) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(static_cast<char *>(chunk_base) + off));
    } else {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(chunk_base, (short)0, 0x7FFFFFFF, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 18);   // sc1 | nt
    }
}

__device__ __forceinline__ float h2f(uint32_t h) {
    const uint16_t b = uint16_t(h);
    _Float16 x;
    __builtin_memcpy(&x, &b, 2);
    return float(x);
}

// high bytes of the four 16-bit values in (a, b), in order
__device__ __forceinline__ uint32_t hi_bytes(uint32_t a, uint32_t b) {
    return ((a >> 8) & 0xFFu) | ((a >> 16) & 0xFF00u) | ((b << 8) & 0xFF0000u) | (b & 0xFF000000u);
}

template <int PATTERN, int U, int POLICY, bool NTL, int LAYOUT>
__global__ __launch_bounds__(kThreads)
void stream_kernel(const void *__restrict__ src, void *__restrict__ dst, int64_t nunits,
                   uint32_t *__restrict__ sink) {
    extern __shared__ uint32_t reserved[];   // occupancy cap only; never touched
    (void)reserved;
    constexpr int64_t kChunk = int64_t(kThreads) * U;
    uint32_t acc = 0;
    for (int64_t c = blockIdx.x; c * kChunk < nunits; c += gridDim.x) {
        const int64_t base = c * kChunk;
        if constexpr (PATTERN == 0) {
            const u32x4 *s = static_cast<const u32x4 *>(src) + base;
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                v[u] = base + i < nunits ? get<NTL>(s + i) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else if constexpr (PATTERN == 1) {
            void *d = static_cast<u32x4 *>(dst) + base;
            const u32x4 v = {uint32_t(c), 1u, 2u, 3u};
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                if (base + i < nunits) put16<POLICY>(d, uint32_t(i) * 16u, v);
            }
        } else if constexpr (PATTERN == 2) {
            const u32x2 *s = static_cast<const u32x2 *>(src) + base;
            void *d = static_cast<f32x4 *>(dst) + base;
            u32x2 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                v[u] = base + i < nunits ? get<NTL>(s + i) : u32x2{0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                const f32x4 y = {h2f(v[u].x & 0xFFFFu), h2f(v[u].x >> 16), h2f(v[u].y & 0xFFFFu),
                                 h2f(v[u].y >> 16)};
                if (base + i < nunits) put16<POLICY>(d, uint32_t(i) * 16u, __builtin_bit_cast(u32x4, y));
            }
        } else if constexpr (PATTERN == 3) {
            const u32x4 *s = static_cast<const u32x4 *>(src) + 2 * base;
            void *d = static_cast<u32x4 *>(dst) + base;
            u32x4 a[U], b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                a[u] = base + i < nunits ? get<NTL>(s + 2 * i) : u32x4{0, 0, 0, 0};
                b[u] = base + i < nunits ? get<NTL>(s + 2 * i + 1) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                const u32x4 o = {hi_bytes(a[u].x, a[u].y), hi_bytes(a[u].z, a[u].w),
                                 hi_bytes(b[u].x, b[u].y), hi_bytes(b[u].z, b[u].w)};
                if (base + i < nunits) put16<POLICY>(d, uint32_t(i) * 16u, o);
            }
        } else if constexpr (PATTERN == 5) {
            const u32x2 *s = static_cast<const u32x2 *>(src) + base;
            void *d = static_cast<u32x4 *>(dst) + base;
            u32x2 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                v[u] = base + i < nunits ? get<NTL>(s + i) : u32x2{0, 0};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                // each byte becomes the high byte of a 16-bit value
                const u32x4 o = {((v[u].x << 8) & 0xFF00u) | ((v[u].x << 16) & 0xFF000000u),
                                 ((v[u].x >> 8) & 0xFF00u) | (v[u].x & 0xFF000000u),
                                 ((v[u].y << 8) & 0xFF00u) | ((v[u].y << 16) & 0xFF000000u),
                                 ((v[u].y >> 8) & 0xFF00u) | (v[u].y & 0xFF000000u)};
                if (base + i < nunits) put16<POLICY>(d, uint32_t(i) * 16u, o);
            }
        } else {
            const uint32_t *s = static_cast<const uint32_t *>(src) + base;
            void *d = static_cast<f32x4 *>(dst) + base;
            uint32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                v[u] = base + i < nunits ? get<NTL>(s + i) : 0u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = LAYOUT == 0 ? u * kThreads + threadIdx.x : threadIdx.x * U + u;
                const f32x4 y = {float(v[u] & 0xFFu), float((v[u] >> 8) & 0xFFu),
                                 float((v[u] >> 16) & 0xFFu), float(v[u] >> 24)};
                if (base + i < nunits) put16<POLICY>(d, uint32_t(i) * 16u, __builtin_bit_cast(u32x4, y));
            }
        }
    }
    if (PATTERN == 0 && acc == 0x9E3779B9u) sink[threadIdx.x] = acc;   // keeps the loads live
}

// elements per unit of each pattern (read/write: bytes per unit)
constexpr int64_t kElemsPerUnit[6] = {16, 16, 4, 16, 4, 8};

template <int PATTERN, int U, bool NTL, int LAYOUT>
hipError_t launch_u(int policy, const void *src, void *dst, int64_t nunits, uint32_t *sink,
                    dim3 grid, unsigned lds, hipStream_t s) {
    if (policy == 0)
        hipLaunchKernelGGL((stream_kernel<PATTERN, U, 0, NTL, LAYOUT>), grid, dim3(kThreads), lds, s, src, dst, nunits, sink);
    else if (policy == 1)
        hipLaunchKernelGGL((stream_kernel<PATTERN, U, 1, NTL, LAYOUT>), grid, dim3(kThreads), lds, s, src, dst, nunits, sink);
    else
        hipLaunchKernelGGL((stream_kernel<PATTERN, U, 2, NTL, LAYOUT>), grid, dim3(kThreads), lds, s, src, dst, nunits, sink);
    return hipGetLastError();
}

template <int PATTERN, int U>
hipError_t launch_l(bool ntl, int layout, int policy, const void *src, void *dst, int64_t nunits,
                    uint32_t *sink, dim3 grid, unsigned lds, hipStream_t s) {
    if (layout == 0)
        return ntl ? launch_u<PATTERN, U, true, 0>(policy, src, dst, nunits, sink, grid, lds, s)
                   : launch_u<PATTERN, U, false, 0>(policy, src, dst, nunits, sink, grid, lds, s);
    return ntl ? launch_u<PATTERN, U, true, 1>(policy, src, dst, nunits, sink, grid, lds, s)
               : launch_u<PATTERN, U, false, 1>(policy, src, dst, nunits, sink, grid, lds, s);
}

template <int PATTERN>
hipError_t launch_p(int unroll, bool ntl, int layout, int policy, const void *src, void *dst,
                    int64_t nunits, uint32_t *sink, unsigned lds, hipStream_t s) {
    int64_t g = (nunits + int64_t(kThreads) * unroll - 1) / (int64_t(kThreads) * unroll);
    if (g < 1) g = 1;
    if (g > kMaxGrid) g = kMaxGrid;
    const dim3 grid((uint32_t)g);
    switch (unroll) {
        case 1: return launch_l<PATTERN, 1>(ntl, layout, policy, src, dst, nunits, sink, grid, lds, s);
        case 2: return launch_l<PATTERN, 2>(ntl, layout, policy, src, dst, nunits, sink, grid, lds, s);
        case 4: return launch_l<PATTERN, 4>(ntl, layout, policy, src, dst, nunits, sink, grid, lds, s);
        default: return launch_l<PATTERN, 8>(ntl, layout, policy, src, dst, nunits, sink, grid, lds, s);
    }
}

}  // namespace

// One launch of pattern `pattern` over n elements (read / write: n bytes)
// on `stream`, in unit layout `layout`, with non-temporal loads when
// nt_loads is 1.  src / dst are device buffers of the pattern's sizes (16-byte
// aligned; dst of pattern 0 is a 1 KiB sink).  n must be a whole number of
// units and below 2^31 units per 16-byte store offset within a chunk (always
// true here).  Returns 0, -1 for bad arguments, or the HIP error code.
extern "C" int gsc_stream(int pattern, const void *src, void *dst, int64_t n, int unroll,
                          int layout, int nt_loads, int policy, int wgs_per_cu, void *stream) {
    if (pattern < 0 || pattern > 5 || n < 0 || policy < 0 || policy > 2 || wgs_per_cu < 0 ||
        (nt_loads != 0 && nt_loads != 1) || (layout != 0 && layout != 1))
        return -1;
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return -1;
    if (n % kElemsPerUnit[pattern] != 0) return -1;
    if ((uintptr_t(src) & 15) || (uintptr_t(dst) & 15)) return -1;
    const int64_t nunits = n / kElemsPerUnit[pattern];
    if (nunits == 0) return 0;
    unsigned lds = 0;
    if (wgs_per_cu > 0) {
        int dev = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess || per_cu <= 0)
            return -1;
        lds = unsigned(per_cu) / unsigned(wgs_per_cu + 1) + 1024u;
        if (lds > 65536u) lds = 65536u;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *sink = static_cast<uint32_t *>(dst);
    hipError_t e;
    switch (pattern) {
        case 0: e = launch_p<0>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
        case 1: e = launch_p<1>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
        case 2: e = launch_p<2>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
        case 3: e = launch_p<3>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
        case 4: e = launch_p<4>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
        default: e = launch_p<5>(unroll, nt_loads == 1, layout, policy, src, dst, nunits, sink, lds, s); break;
    }
    return e == hipSuccess ? 0 : int(e);
}
