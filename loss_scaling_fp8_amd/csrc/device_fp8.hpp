// device_fp8.hpp -- gfx950 device helpers for the OCP FP8 cast and its
// inverse, used by the quantize and dequantize kernels.
//
// Formats ("Numerical Precision, Mixed Precision, and Loss Scaling", FP8
// specification paragraph): E4M3 has exponent bias 7, 3 fraction bits, max
// normal 448, no infinities and a single NaN fraction pattern (S.1111.111);
// E5M2 has bias 15, 2 fraction bits, max normal 57344 and IEEE-style
// infinities and NaNs.
//
// The cast ("Mixed precision and FP8 training", FP8 training section,
// quant() of fp8_scaling.py): divide by the scale, clamp to [-MAX, MAX],
// round to the nearest FP8 value with ties to an even fraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsk {

template <int FMT> struct Fp8;

template <> struct Fp8<0> {                           // OCP E4M3
    static constexpr uint32_t kMaxBits = 0x43E00000u;       // 448.0f
    static constexpr float kMax = 448.0f;
    static constexpr uint32_t kMinNormalBits = 0x3C800000u; // 2^-6
    static constexpr int kDrop = 20;                        // 23 - 3 fraction bits
    static constexpr uint32_t kRebias = (127u - 7u) << 23;  // FP32 -> FP8 exponent
    static constexpr float kSubAnchor = 16384.0f;           // 2^14, FP32 ulp 2^-9
};

template <> struct Fp8<1> {                           // OCP E5M2
    static constexpr uint32_t kMaxBits = 0x47600000u;       // 57344.0f
    static constexpr float kMax = 57344.0f;
    static constexpr uint32_t kMinNormalBits = 0x38800000u; // 2^-14
    static constexpr int kDrop = 21;                        // 23 - 2 fraction bits
    static constexpr uint32_t kRebias = (127u - 15u) << 23;
    static constexpr float kSubAnchor = 128.0f;             // 2^7, FP32 ulp 2^-16
};

__device__ __forceinline__ float as_f32(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// FP8 magnitude code (0 .. max code) of a non-negative, non-NaN FP32 value
// given by its bits `b` (Inf and anything above MAX saturate).
//  - Normal FP8 range: drop the extra FP32 fraction bits with
//    round-to-nearest-even; a carry out of the fraction lands in the
//    exponent field, which is exactly the next FP8 code.
//  - Below the smallest FP8 normal: adding an anchor whose FP32 ulp equals
//    the FP8 subnormal spacing makes the FP32 adder itself round the value
//    to that spacing (ties to even); the difference of the bit patterns is
//    the subnormal code (the top value is the smallest normal's code).
template <int FMT>
__device__ __forceinline__ uint32_t encode_mag(uint32_t b) {
    using T = Fp8<FMT>;
    b = b < T::kMaxBits ? b : T::kMaxBits;
    const uint32_t lsb = (b >> T::kDrop) & 1u;
    const uint32_t normal =
        (b - T::kRebias + ((1u << (T::kDrop - 1)) - 1u) + lsb) >> T::kDrop;
    const uint32_t sub = as_u32(as_f32(b) + T::kSubAnchor) - as_u32(T::kSubAnchor);
    return b < T::kMinNormalBits ? sub : normal;
}

// Full code of x / s for any FP32 x and s (IEEE division), following the
// cast definition: NaN x -> sign|0x7F; NaN quotient -> 0x7F; otherwise the
// sign of the quotient with the saturated, rounded magnitude.
template <int FMT>
__device__ __forceinline__ uint32_t cast_exact(float x, float s) {
    const uint32_t xb = as_u32(x);
    if (__builtin_isnan(x)) return ((xb >> 24) & 0x80u) | 0x7Fu;
    const float y = x / s;
    if (__builtin_isnan(y)) return 0x7Fu;
    const uint32_t yb = as_u32(y);
    return ((yb >> 24) & 0x80u) | encode_mag<FMT>(yb & 0x7FFFFFFFu);
}

// |x| / s for finite |x| >= 0 and s in the "fast" range [2^-80, 2^126],
// from r = fl32(1/s): q0 = |x| r, then one FMA correction with the exact
// remainder |x| - q0 s.  Equal to fl32(|x| / s) whenever the quotient is at
// least 2^-20 (no underflow in the remainder), and below 2^-19 whenever the
// true quotient is below 2^-20, so the FP8 code always equals that of the
// correctly rounded quotient.
__device__ __forceinline__ float div_by_scale(float ax, float s, float r) {
    const float q0 = ax * r;
    const float e = __builtin_fmaf(-q0, s, ax);
    return __builtin_fmaf(e, r, q0);
}

// Scales for which div_by_scale is used: 2^-80 <= s <= 2^126 (positive,
// normal, with a normal reciprocal).  Every scale derived from a block amax
// (>= 1e-12 / 57344, <= FLT_MAX / 448) is in this range.
__device__ __forceinline__ bool fast_scale(float s) {
    return (as_u32(s) - 0x17800000u) <= (0x7E800000u - 0x17800000u);
}

// Exact FP32 value of an FP8 code.
template <int FMT> __device__ __forceinline__ float decode(uint32_t c);

template <> __device__ __forceinline__ float decode<0>(uint32_t c) {
    const uint32_t m = c & 0x7Fu;
    const uint32_t sign = (c & 0x80u) << 24;
    // subnormals (exponent field 0): m * 2^-9; normals: rebias the exponent
    const float sub = (float)m * 0x1p-9f;
    const uint32_t mag = m < 8u ? as_u32(sub) : (m << 20) + Fp8<0>::kRebias;
    const uint32_t bits = (m == 0x7Fu) ? 0x7FC00000u : (mag | sign);
    return as_f32(bits);
}

template <> __device__ __forceinline__ float decode<1>(uint32_t c) {
    // E5M2 has FP16's sign, exponent width and bias: it is the upper byte of
    // an FP16 encoding, and FP16 -> FP32 widening is exact (subnormals,
    // infinities and NaNs included).
    const _Float16 h = __builtin_bit_cast(_Float16, (unsigned short)((c & 0xFFu) << 8));
    return (float)h;
}

// FP32 result written for a dequantized value: canonical NaN for any NaN.
__device__ __forceinline__ float canon(float v) {
    return __builtin_isnan(v) ? as_f32(0x7FC00000u) : v;
}

// ---- lane exchange (DPP) for reductions inside groups of 2^k lanes
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
}
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
}
__device__ __forceinline__ uint32_t dpp_mirror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false); // row_mirror
}

// max over groups of G consecutive lanes (G = 1, 2, 4, 8, 16), all active
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    if (G >= 2) v = max(v, dpp_xor1(v));
    if (G >= 4) v = max(v, dpp_xor2(v));
    if (G >= 8) v = max(v, dpp_half_mirror(v));
    if (G >= 16) v = max(v, dpp_mirror(v));
    return v;
}

// max over the whole 64-lane wave (all lanes active)
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = group_max<16>(v);
    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

}  // namespace gsk
