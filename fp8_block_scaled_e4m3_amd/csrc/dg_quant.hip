// dg_quant.hip -- gfx950 kernels that cast fp32 / bf16 matrices to E4M3 (or E5M2)
// with the fine-grained scales the GEMM consumes.
//
// The README ("DeepGEMM: clean and efficient FP8 GEMM kernels", nipponese.news
// translation, usage paragraph) leaves the FP8 cast and the transposition of the
// LHS scales to a prior kernel; these are that kernel, producing exactly the
// layouts dg_gemm_fp8_nt reads:
//   1x128  : one scale per (row, 128-wide K block), written MN-major sa[kb*ld_sa + row]
//   128x128: one scale per (128-row block, 128-wide K block), written sb[rb*(K/128) + kb]
// Per block: amax = max |x| (NaN entries do not raise it), scale = fp32(amax / 448)
// (1 when amax is 0), q = E4M3 round-to-nearest-even of fp32(x / scale), saturating
// at +-448 (the format's largest finite value), NaN -> 0x7F, sign of zero kept.
// E5M2 output (the blog's other FP8 format, hnwysp.cn section 2.3) is the same with
// 57344, E5M2's largest finite value, in place of 448.
// Both divisions are IEEE-correctly-rounded fp32 divisions, so the codes are a
// deterministic function of the input.  Each kernel reads its input once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {

namespace {

constexpr int kQBlock = 128;
constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);   // bf16 -> fp32 is exact
}

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

// One 16-byte load: 4 fp32 or 8 bf16 values, widened to fp32 (bf16 -> fp32 is exact).
template <typename T> struct Vec;
template <> struct Vec<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float* p, float* v) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 t = __builtin_nontemporal_load((const f4*)p);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
};
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
        typedef unsigned u4 __attribute__((ext_vector_type(4)));
        const u4 t = __builtin_nontemporal_load((const u4*)p);
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};

__device__ __forceinline__ float amax_of(const float* v, int n, float amax) {
    for (int i = 0; i < n; ++i) {
        const float m = fabsf(v[i]);
        amax = m > amax ? m : amax;              // a NaN never raises the maximum
    }
    return amax;
}

// Scales whose reciprocal is a normal number: the fast quotient below is exact there.
__device__ __forceinline__ bool fast_scale(float scale) { return scale > 0x1p-125f && scale < 0x1p125f; }

// RN(1/s) for 2^-125 < s < 2^125 (the fast path's scales): one FMA Newton step from the
// hardware reciprocal.  An exhaustive run on gfx950 over every fp32 significand at every
// exponent of that range matched the IEEE division bit for bit.
__device__ __forceinline__ float rcp_exact(float s) {
    const float y = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
}

// x / scale correctly rounded, given r = RN(1/scale) with scale and r normal:
// q = RN(x*r) is within one ulp of the quotient, the residual x - q*scale is exact
// in a fused multiply-add, and one correction step rounds correctly (Markstein's
// theorem for radix-2 division).  The quotient has the sign of x (scale > 0); the
// copysign keeps it for x = -0, where the correction step would return +0.
__device__ __forceinline__ float div_fast(float x, float scale, float r) {
    const float q = x * r;
    const float e = __builtin_fmaf(-q, scale, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), x);
}

// fp32(amax / FMAX) (1 when amax is 0), correctly rounded: with the constant r = RN(1/FMAX),
// q = RN(amax r), the residual amax - q FMAX exact in an FMA and one correction step give
// the correctly rounded quotient while it is a normal number (the step div_fast uses,
// here with a fixed divisor; checked against exact rational division on 4e4 values per
// format across the range).  Smaller or infinite amax take the IEEE division.
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

// N codes of v / scale packed little-endian (4 -> one dword, 8 -> two).  Fast path
// (every value of the wave finite or infinite but not NaN, the scale in range): the
// quotient as above and gfx950's FP8 convert (E4M3 or E5M2), which rounds to nearest
// even with subnormals and, for the magnitudes here (|q| at most the format's
// largest value up to one rounding), agrees with the software encoder.  Otherwise
// each code is computed in software with an IEEE division.
template <int N, int FMT>
__device__ __forceinline__ void store_codes(uint8_t* dst, const float* v, float scale, bool fast) {
    using F = Fp8Out<FMT>;
    uint32_t w[N / 4];
    if (fast) {
        const float r = rcp_exact(scale);
#pragma unroll
        for (int d = 0; d < N / 4; ++d) {
            int c = F::template pack<false>(div_fast(v[4 * d], scale, r), div_fast(v[4 * d + 1], scale, r), 0);
            c = F::template pack<true>(div_fast(v[4 * d + 2], scale, r), div_fast(v[4 * d + 3], scale, r), c);
            w[d] = (uint32_t)c;
        }
    } else {
#pragma unroll
        for (int d = 0; d < N / 4; ++d) {
            uint32_t c = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) c |= F::code(v[4 * d + e] / scale) << (8 * e);
            w[d] = c;
        }
    }
    if constexpr (N == 4) *(uint32_t*)dst = w[0];
    else *(uint2*)dst = uint2{w[0], w[1]};
}

// true when any of the n values is a NaN
__device__ __forceinline__ bool any_nan(const float* v, int n) {
    bool r = false;
    for (int i = 0; i < n; ++i) r |= v[i] != v[i];
    return r;
}

// one decision for the whole wave, so the paths never diverge inside it
__device__ __forceinline__ bool wave_all(bool b) { return __ballot(!b) == 0; }

// Unsigned 32-bit division by a divisor fixed for the launch, as a multiply-high and
// shifts (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, the round-up method): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (t + ((n - t) >> 1)) >> (l - 1) for
// t = mulhi(n, m) and every 32-bit n; d = 1 uses m = 0 and no shifts.
struct DivU32 {
    uint32_t m, s1, s2;
};
__host__ DivU32 make_div_u32(uint32_t d) {
    if (d <= 1) return DivU32{0u, 0u, 0u};
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = (((1ull << 32) * ((1ull << l) - d)) / d) + 1;
    return DivU32{(uint32_t)m, 1u, l - 1};
}
__device__ __forceinline__ uint32_t div_u32(uint32_t n, DivU32 f) {
    const uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// 1x128: a 128-element row block is read by L = 128/N lanes with one 16-byte load
// each (the block's bytes are contiguous, so every load instruction is coalesced).
// A thread handles kRowsPerThread row blocks of one K block, their loads all in
// flight before any is reduced.  Blocks are numbered K block fastest, so a
// workgroup reads long contiguous stretches of each row.
constexpr int kRowsPerThread = 4;

template <typename T, int FMT>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const T* __restrict__ x, long ldx, int rows, int kblocks, DivU32 kdiv, uint8_t* __restrict__ q,
                   long ldq, float* __restrict__ sa, long ld_sa) {
    constexpr int N = Vec<T>::N, L = kQBlock / N, GPW = 256 / L;   // groups of L lanes per workgroup
    const int lg = threadIdx.x % L, grp = threadIdx.x / L;
    // workgroup w handles groups [w*GPW*R, (w+1)*GPW*R); group g = (row, kb) with kb
    // fastest (the host keeps rows * kblocks below 2^31)
    const unsigned groups_total = (unsigned)rows * (unsigned)kblocks;
    const unsigned g0 = blockIdx.x * (unsigned)(GPW * kRowsPerThread) + grp;
    float v[kRowsPerThread][N];
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
        const unsigned g = g0 + r * GPW;
        if (g < groups_total) {
            const unsigned row = div_u32(g, kdiv), kb = g - row * (unsigned)kblocks;
            Vec<T>::load(x + (long)row * ldx + kb * kQBlock + lg * N, v[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerThread; ++r) {
        const unsigned g = g0 + r * GPW;
        if (g >= groups_total) break;                   // uniform over the L lanes of a group
        float amax = amax_of(v[r], N, 0.f);
#pragma unroll
        for (int off = L / 2; off >= 1; off >>= 1) {
            const float o = __shfl_xor(amax, off, L);
            amax = o > amax ? o : amax;
        }
        const float scale = block_scale<FMT>(amax);
        const unsigned row = div_u32(g, kdiv), kb = g - row * (unsigned)kblocks;
        const bool fast = wave_all(fast_scale(scale) && !any_nan(v[r], N));
        store_codes<N, FMT>(q + (long)row * ldq + kb * kQBlock + lg * N, v[r], scale, fast);
        if (lg == 0) sa[(long)kb * ld_sa + row] = scale;
    }
}

// 128x128: one workgroup per block.  Every load instruction of the workgroup reads
// whole 512-byte (fp32) or 256-byte (bf16) row segments: lane t of a pass covers
// row pass*RPP + t/L, columns (t%L)*N .. +N.  All passes' loads are in flight
// before the reduction.
template <typename T, int FMT>
__global__ void __launch_bounds__(256)
quant_128x128_kernel(const T* __restrict__ x, long ldx, int rows, int kblocks, uint8_t* __restrict__ q, long ldq,
                     float* __restrict__ sb) {
    constexpr int N = Vec<T>::N, L = kQBlock / N, RPP = 256 / L, PASSES = kQBlock / RPP;
    __shared__ float s_amax[4];
    const int kb = blockIdx.x, rb = blockIdx.y;
    const int t = threadIdx.x;
    const int r0 = rb * kQBlock + t / L;
    const long c0 = (long)kb * kQBlock + (t % L) * N;
    float v[PASSES][N];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int row = r0 + i * RPP;
        if (row < rows) Vec<T>::load(x + (long)row * ldx + c0, v[i]);
        else
#pragma unroll
            for (int e = 0; e < N; ++e) v[i][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) amax = amax_of(v[i], N, amax);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(amax, off, 64);
        amax = o > amax ? o : amax;
    }
    if ((t & 63) == 0) s_amax[t >> 6] = amax;
    __syncthreads();
    amax = s_amax[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) amax = s_amax[w] > amax ? s_amax[w] : amax;
    const float scale = block_scale<FMT>(amax);
    if (t == 0) sb[(long)rb * kblocks + kb] = scale;
    bool nan = false;
#pragma unroll
    for (int i = 0; i < PASSES; ++i) nan |= any_nan(v[i], N);
    const bool fast = wave_all(fast_scale(scale) && !nan);
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int row = r0 + i * RPP;
        if (row < rows) store_codes<N, FMT>(q + (long)row * ldq + c0, v[i], scale, fast);
    }
}

}  // namespace

namespace {

template <int FMT>
hipError_t launch_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                        long ld_sa, hipStream_t stream) {
    const int kblocks = k / kQBlock;
    const DivU32 kdiv = make_div_u32((uint32_t)kblocks);
    const long per_wg = (x_bf16 ? 256 / 16 : 256 / 32) * (long)kRowsPerThread;   // groups per workgroup
    // row chunks small enough for 32-bit group indices inside the kernel
    const long chunk = ((1l << 30) / kblocks) > 0 ? ((1l << 30) / kblocks) : 1;
    for (long r0 = 0; r0 < rows; r0 += chunk) {
        const int nr = (int)(rows - r0 < chunk ? rows - r0 : chunk);
        const long blocks = ((long)nr * kblocks + per_wg - 1) / per_wg;
        if (x_bf16)
            hipLaunchKernelGGL((quant_1x128_kernel<uint16_t, FMT>), dim3((unsigned)blocks), dim3(256), 0, stream,
                               static_cast<const uint16_t*>(x) + r0 * ldx, ldx, nr, kblocks, kdiv, q + r0 * ldq,
                               ldq, sa + r0, ld_sa);
        else
            hipLaunchKernelGGL((quant_1x128_kernel<float, FMT>), dim3((unsigned)blocks), dim3(256), 0, stream,
                               static_cast<const float*>(x) + r0 * ldx, ldx, nr, kblocks, kdiv, q + r0 * ldq, ldq,
                               sa + r0, ld_sa);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int FMT>
hipError_t launch_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sb,
                          hipStream_t stream) {
    const int kblocks = k / kQBlock;
    const dim3 grid((unsigned)kblocks, (unsigned)((rows + kQBlock - 1) / kQBlock));
    if (x_bf16)
        hipLaunchKernelGGL((quant_128x128_kernel<uint16_t, FMT>), grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), ldx, rows, kblocks, q, ldq, sb);
    else
        hipLaunchKernelGGL((quant_128x128_kernel<float, FMT>), grid, dim3(256), 0, stream,
                           static_cast<const float*>(x), ldx, rows, kblocks, q, ldq, sb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                              long ld_sa, int q_e5m2, hipStream_t stream) {
    return q_e5m2 ? launch_1x128<1>(x, x_bf16, ldx, rows, k, q, ldq, sa, ld_sa, stream)
                  : launch_1x128<0>(x, x_bf16, ldx, rows, k, q, ldq, sa, ld_sa, stream);
}

hipError_t launch_quant_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq,
                                float* sb, int q_e5m2, hipStream_t stream) {
    return q_e5m2 ? launch_128x128<1>(x, x_bf16, ldx, rows, k, q, ldq, sb, stream)
                  : launch_128x128<0>(x, x_bf16, ldx, rows, k, q, ldq, sb, stream);
}

}  // namespace dg
