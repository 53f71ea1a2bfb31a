// device.hpp -- gfx950 device helpers shared by the libw8a8 kernels:
// vector types, element loads, the quantisation of one element, output
// conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// Same numbering as the public enums in w8a8.h.
enum QType { Q_INT8 = 0, Q_FP8 = 1 };
enum DType { D_BF16 = 0, D_FP16 = 1, D_F32 = 2, D_I32 = 3 };

template <int QT>
struct QMax;
template <>
struct QMax<Q_FP8> {
    static constexpr float value = 448.0f;  // e4m3 max-norm
};
template <>
struct QMax<Q_INT8> {
    static constexpr float value = 127.0f;  // symmetric int8
};

// ------------------------------------------------------------------ loads
// Eight consecutive high-precision elements starting at element `idx`
// (16-byte aligned for 2-byte types, 32-byte for float32), widened to float.
// NT: non-temporal loads, for data read once (the stream does not evict
// reused lines); else cached, for data that a later pass reads again.
template <typename T>
__device__ __forceinline__ T load16(const T* p, bool nt) {
    return nt ? __builtin_nontemporal_load(p) : *p;
}
// The same in two halves: the raw 16 (float32: 32) bytes, then their
// widening, so that several loads can be in flight before the first use.
template <int XT, bool NT = true>
__device__ __forceinline__ void load8_raw(const void* base, int64_t idx, u32x4 r[2]) {
    if constexpr (XT == D_F32) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(base) + idx);
        r[0] = load16(p, NT);
        r[1] = load16(p + 1, NT);
    } else {
        r[0] = load16(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx), NT);
    }
}
template <int XT>
__device__ __forceinline__ void widen8(const u32x4 r[2], float v[8]) {
    if constexpr (XT == D_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(r[0][i] << 16);
            v[2 * i + 1] = __uint_as_float(r[0][i] & 0xFFFF0000u);
        }
    } else if constexpr (XT == D_FP16) {
        const h16x8 h = __builtin_bit_cast(h16x8, r[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(h[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(r[0][i]);
            v[4 + i] = __uint_as_float(r[1][i]);
        }
    }
}
template <int XT, bool NT = true>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float v[8]) {
    u32x4 r[2];
    load8_raw<XT, NT>(base, idx, r);
    widen8<XT>(r, v);
}

// ----------------------------------------------------------- quantisation
// Correctly rounded binary32 quotient x / s, given r = 1/s rounded to double.
//
// Why this is exact: x*r in double carries a relative error below 2^-52
// (one rounding in r, one in the product). For x, s in binary32, x / s can
// come within relative distance 2^-49 of a binary32 rounding boundary
// (a midpoint t = odd * 2^e with a 25-bit odd part) only by hitting it, since
// x - s*t is a non-zero multiple of the last bit of s*t, whose significand
// has at most 49 bits; and it cannot hit it, because the 25-bit odd part of
// t would have to divide into the at most 24-bit odd part of x. So rounding
// the double product to binary32 gives the same result as rounding the exact
// quotient: the IEEE division the quantisation is defined with, at the cost
// of one multiply and two conversions per element.
__device__ __forceinline__ float div_rn(float x, double r) {
    return static_cast<float>(static_cast<double>(x) * r);
}

// Four fp8 e4m3 codes, packed little-endian. Saturate at +-448 first: the
// hardware conversion rounds to nearest even but turns values beyond the
// format's range into NaN. NaN becomes 0x7F.
__device__ __forceinline__ uint32_t enc4_fp8(float t0, float t1, float t2, float t3) {
    float c0 = fminf(fmaxf(t0, -448.0f), 448.0f);
    float c1 = fminf(fmaxf(t1, -448.0f), 448.0f);
    float c2 = fminf(fmaxf(t2, -448.0f), 448.0f);
    float c3 = fminf(fmaxf(t3, -448.0f), 448.0f);
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
    uint32_t nan = (t0 != t0 ? 0x000000FFu : 0u) | (t1 != t1 ? 0x0000FF00u : 0u) |
                   (t2 != t2 ? 0x00FF0000u : 0u) | (t3 != t3 ? 0xFF000000u : 0u);
    return (w & ~nan) | (0x7F7F7F7Fu & nan);
}

// Symmetric int8: round half to even, clamp to [-127, 127]; NaN becomes 0.
__device__ __forceinline__ uint32_t enc1_i8(float t) {
    float r = fminf(fmaxf(__builtin_rintf(t), -127.0f), 127.0f);
    int i = (t != t) ? 0 : static_cast<int>(r);
    return static_cast<uint32_t>(i) & 0xFFu;
}

__device__ __forceinline__ uint32_t enc4_i8(float t0, float t1, float t2, float t3) {
    return enc1_i8(t0) | (enc1_i8(t1) << 8) | (enc1_i8(t2) << 16) | (enc1_i8(t3) << 24);
}

// Quantise 8 elements with the per-group reciprocal r = 1/s (double).
template <int QT>
__device__ __forceinline__ u32x2 quant8(const float v[8], double r) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = div_rn(v[i], r);
    u32x2 out;
    if constexpr (QT == Q_FP8) {
        out[0] = enc4_fp8(t[0], t[1], t[2], t[3]);
        out[1] = enc4_fp8(t[4], t[5], t[6], t[7]);
    } else {
        out[0] = enc4_i8(t[0], t[1], t[2], t[3]);
        out[1] = enc4_i8(t[4], t[5], t[6], t[7]);
    }
    return out;
}

// The group scale: absmax / Qmax in binary32 (an IEEE division); 1.0 for an
// all-zero group.
template <int QT>
__device__ __forceinline__ float scale_from_absmax(float amax) {
    return amax == 0.0f ? 1.0f : amax / QMax<QT>::value;
}

template <int QT>
__host__ __device__ constexpr float scale_of_zero() {
    return 1.0f;  // the scale of an all-zero group (scale_from_absmax(0))
}

// --------------------------------------------------------- output stores
// The float argument is first pinned in a register: otherwise instruction
// selection folds a preceding float multiply into the narrowing conversion
// (v_fma_mix with a +0 addend), which rounds the exact product only once and
// turns -0 into +0, where the definition rounds to binary32 first.
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
    asm volatile("" : "+v"(f));
    __bf16 h = static_cast<__bf16>(f);  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t to_fp16_bits(float f) {
    asm volatile("" : "+v"(f));
    _Float16 h = static_cast<_Float16>(f);  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// --------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

}  // namespace w8a8
