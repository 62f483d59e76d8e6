// dg_cast_math.h -- scalar arithmetic of the FP8 casts (device code): the
// round-to-nearest-even FP8 encoders, the block scale fp32(amax / FP8 max), and the
// correctly rounded quotient x / scale of the fast path.  Included by the cast kernels
// and by the test probe that checks these functions exhaustively; nothing else.
//
// The rule implemented (a reading of the "DeepGEMM" README's usage paragraph, which
// leaves the cast to a prior kernel, with DeepSeek-V3's fine-grained scale blocks):
// scale = fp32(amax / FMAX) (1 when amax is 0), code = FP8 RNE of fp32(x / scale)
// saturating at +-FMAX, NaN -> 0x7F, sign of zero kept; FMAX is 448 for E4M3 and
// 57344 for E5M2 (the blog's two FP8 formats, hnwysp.cn section 2.3).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {
namespace castmath {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

// E4M3 code of an fp32 value, round to nearest even, saturating.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(y);
    if (!(a == a)) return 0x7Fu;                       // NaN
    if (a >= kE4M3Max) return sign | 0x7Eu;            // saturate at 448
    if (a < 0.015625f) {                               // below 2^-6: multiples of 2^-9
        const float q = __builtin_rintf(a * 512.0f);   // exact scaling, RNE (q <= 8)
        return sign | (uint32_t)q;                     // q == 8 is the smallest normal
    }
    // normal range: keep 3 of 23 mantissa bits, ties to even, carry into the exponent
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const uint32_t rounded = ab + 0x7FFFFu + ((ab >> 20) & 1u);
    return sign | ((rounded >> 20) - (120u << 3));     // rebias exponent 127 -> 7
}

// E5M2 code of an fp32 value, round to nearest even, saturating (bias 15, two
// stored mantissa bits, subnormals are the multiples of 2^-16 below 2^-14).
__device__ __forceinline__ uint32_t e5m2_code(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = fabsf(y);
    if (!(a == a)) return 0x7Fu;                       // NaN
    if (a >= kE5M2Max) return sign | 0x7Bu;            // saturate at 57344
    if (a < 0x1p-14f) {                                // below 2^-14: multiples of 2^-16
        const float q = __builtin_rintf(a * 65536.0f); // exact scaling, RNE (q <= 4)
        return sign | (uint32_t)q;                     // q == 4 is the smallest normal
    }
    // normal range: keep 2 of 23 mantissa bits, ties to even, carry into the exponent
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const uint32_t rounded = ab + 0xFFFFFu + ((ab >> 21) & 1u);
    return sign | ((rounded >> 21) - (112u << 2));     // rebias exponent 127 -> 15
}

// Output format FMT: 0 = E4M3, 1 = E5M2.
template <int FMT> struct Fp8Out;
template <> struct Fp8Out<0> {
    static constexpr float kMax = kE4M3Max;
    static __device__ __forceinline__ uint32_t code(float y) { return e4m3_code(y); }
    template <bool HI>
    static __device__ __forceinline__ int pack(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
    }
};
template <> struct Fp8Out<1> {
    static constexpr float kMax = kE5M2Max;
    static __device__ __forceinline__ uint32_t code(float y) { return e5m2_code(y); }
    template <bool HI>
    static __device__ __forceinline__ int pack(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    }
};

// Scales the fast quotient below is exact for: 2^-64 <= scale < 2^125.  Above, the
// reciprocal would not be a normal number.  Below, the residual x - q*scale of a
// quotient q that still matters for a code (|q| >= 2^-17, half the smallest E5M2
// subnormal; 2^-10 for E4M3) could fall under fp32's subnormal granularity and be
// rounded; from 2^-64 up it is a multiple of ulp(q)*ulp(scale) >= 2^-40 * 2^-87, well
// above 2^-149, so it is exact.  Smaller scales take the software path.
__device__ __forceinline__ bool fast_scale(float scale) { return scale >= 0x1p-64f && scale < 0x1p125f; }

// RN(1/s) for the fast path's scales (2^-64 <= s < 2^125): one FMA Newton step from the
// hardware reciprocal estimate.  A GPU test runs it over every fp32 value of that range
// against the IEEE division, bit for bit.
__device__ __forceinline__ float rcp_exact(float s) {
    const float y = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
}

// x / scale correctly rounded, given r = RN(1/scale) for a scale the fast path admits:
// q = RN(x*r) is within one ulp of the quotient, the residual x - q*scale is exact
// in a fused multiply-add (see fast_scale for the small scales), and one correction
// step rounds correctly (Markstein's theorem for radix-2 division).  A quotient below
// fp32's normal range may come out inexact, but it lies far under half the smallest
// FP8 subnormal, so its code is a zero of the right sign either way.  The quotient has
// the sign of x (scale > 0); the copysign keeps it for x = -0, where the correction
// step would return +0.
__device__ __forceinline__ float div_fast(float x, float scale, float r) {
    const float q = x * r;
    const float e = __builtin_fmaf(-q, scale, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), x);
}

// fp32(amax / FMAX) (1 when amax is 0), correctly rounded: with the constant r = RN(1/FMAX),
// q = RN(amax r), the residual amax - q FMAX exact in an FMA and one correction step give
// the correctly rounded quotient while it is a normal number (the step div_fast uses,
// here with a fixed divisor; a CPU test replays this arithmetic for every fp32 amax of
// the range, in both formats, against the IEEE division).  Smaller or infinite amax take
// the IEEE division.
template <int FMT>
__device__ __forceinline__ float block_scale(float amax) {
    constexpr float b = Fp8Out<FMT>::kMax;
    constexpr float r = 1.0f / b;
    if (amax == 0.f) return 1.f;
    if (!(amax >= b * 0x1p-125f && amax <= 0x1p127f)) return amax / b;
    const float q = amax * r;
    const float e = __builtin_fmaf(-q, b, amax);
    return __builtin_fmaf(e, r, q);
}

}  // namespace castmath
}  // namespace dg
