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
};

template <> struct Fp8<1> {                           // OCP E5M2
    static constexpr uint32_t kMaxBits = 0x47600000u;       // 57344.0f
    static constexpr float kMax = 57344.0f;
};

__device__ __forceinline__ float as_f32(uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// Round-to-nearest-even FP32 -> FP8 by gfx950's OCP conversion, two values
// per instruction, into the low (HI = false) or high 16 bits of `old`.
// Black-box checked over all 2^32 FP32 inputs of both formats: for every
// non-NaN input within [-MAX, MAX] it returns exactly the code of the
// format definition (subnormals, ties to even, the sign of zero); values
// above MAX but below the next would-be FP8 value's midpoint (E4M3: 464,
// E5M2: 61440) also give the MAX code.  NaN inputs are never passed (their
// sign and payload rules differ), nor larger magnitudes (they give NaN/Inf).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b, uint32_t old) {
    if constexpr (FMT == 0)
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else
        return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

template <int FMT>
__device__ __forceinline__ float clamp_max(float y) {     // y not NaN
    return __builtin_fabsf(y) > Fp8<FMT>::kMax ? __builtin_copysignf(Fp8<FMT>::kMax, y) : y;
}

// Full code of x / s for any FP32 x and s (IEEE division), following the
// cast definition: NaN x -> sign|0x7F; NaN quotient -> 0x7F; otherwise the
// quotient clamped to [-MAX, MAX] and rounded to nearest even (sign kept).
template <int FMT>
__device__ __forceinline__ uint32_t cast_exact(float x, float s) {
    if (__builtin_isnan(x)) return ((as_u32(x) >> 24) & 0x80u) | 0x7Fu;
    const float y = x / s;
    if (__builtin_isnan(y)) return 0x7Fu;
    return cvt_pk<FMT, false>(clamp_max<FMT>(y), 0.0f, 0u) & 0xFFu;
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

// Exact FP32 values of the four FP8 codes packed in a 32-bit word (byte 0
// first), by gfx950's OCP FP8 -> FP32 conversion.  Every non-NaN code
// converts exactly (checked for all 256 codes of both formats against the
// format definition); NaN codes give a NaN, which callers canonicalise.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int FMT>
__device__ __forceinline__ void decode4(uint32_t w, float (&v)[4]) {
    f32x2_t lo, hi;
    if constexpr (FMT == 0) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    }
    v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
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
