// dg_quant.hip -- gfx950 kernels that cast fp32 / bf16 matrices to E4M3 with the
// fine-grained scales the GEMM consumes.
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
// Both divisions are IEEE-correctly-rounded fp32 divisions, so the codes are a
// deterministic function of the input.  Each kernel reads its input once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {

namespace {

constexpr int kQBlock = 128;
constexpr float kE4M3Max = 448.0f;

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

// 16 lanes per (row, K block): each lane owns 8 consecutive elements.
template <typename T>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const T* __restrict__ x, long ldx, int rows, int kblocks, uint8_t* __restrict__ q, long ldq,
                   float* __restrict__ sa, long ld_sa) {
    const long blk = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;   // row fastest
    if (blk >= (long)rows * kblocks) return;                         // whole 16-lane groups
    const int l16 = threadIdx.x & 15;
    const int row = (int)(blk % rows), kb = (int)(blk / rows);
    const long k0 = (long)kb * kQBlock + l16 * 8;
    const T* src = x + (long)row * ldx + k0;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = load_elem(src + i);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float m = fabsf(v[i]);
        amax = m > amax ? m : amax;
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        const float o = __shfl_xor(amax, off, 16);
        amax = o > amax ? o : amax;
    }
    const float scale = amax == 0.f ? 1.f : amax / kE4M3Max;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_code(v[i] / scale) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_code(v[4 + i] / scale) << (8 * i);
    *(uint2*)(q + (long)row * ldq + k0) = uint2{lo, hi};
    if (l16 == 0) sa[(long)kb * ld_sa + row] = scale;
}

// One workgroup per 128x128 block: thread t owns row t/2, columns (t%2)*64 .. +63.
template <typename T>
__global__ void __launch_bounds__(256)
quant_128x128_kernel(const T* __restrict__ x, long ldx, int rows, int kblocks, uint8_t* __restrict__ q, long ldq,
                     float* __restrict__ sb) {
    __shared__ float s_amax[4];
    const int kb = blockIdx.x, rb = blockIdx.y;
    const int t = threadIdx.x;
    const int row = rb * kQBlock + (t >> 1);
    const long c0 = (long)kb * kQBlock + (t & 1) * 64;
    const bool live = row < rows;
    float v[64];
    float amax = 0.f;
    if (live) {
        const T* src = x + (long)row * ldx + c0;
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = load_elem(src + i);
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const float m = fabsf(v[i]);
            amax = m > amax ? m : amax;
        }
    }
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
    const float scale = amax == 0.f ? 1.f : amax / kE4M3Max;
    if (t == 0) sb[(long)rb * kblocks + kb] = scale;
    if (!live) return;
    uint8_t* dst = q + (long)row * ldq + c0;
#pragma unroll
    for (int i = 0; i < 64; i += 8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= e4m3_code(v[i + e] / scale) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= e4m3_code(v[i + 4 + e] / scale) << (8 * e);
        *(uint2*)(dst + i) = uint2{lo, hi};
    }
}

}  // namespace

hipError_t launch_quant_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                              long ld_sa, hipStream_t stream) {
    const int kblocks = k / kQBlock;
    const long groups = (long)rows * kblocks;
    const long blocks = (groups * 16 + 255) / 256;
    if (x_bf16)
        hipLaunchKernelGGL(quant_1x128_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), ldx, rows, kblocks, q, ldq, sa, ld_sa);
    else
        hipLaunchKernelGGL(quant_1x128_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const float*>(x), ldx, rows, kblocks, q, ldq, sa, ld_sa);
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq,
                                float* sb, hipStream_t stream) {
    const int kblocks = k / kQBlock;
    const dim3 grid((unsigned)kblocks, (unsigned)((rows + kQBlock - 1) / kQBlock));
    if (x_bf16)
        hipLaunchKernelGGL(quant_128x128_kernel<uint16_t>, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), ldx, rows, kblocks, q, ldq, sb);
    else
        hipLaunchKernelGGL(quant_128x128_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(x),
                           ldx, rows, kblocks, q, ldq, sb);
    return hipGetLastError();
}

}  // namespace dg
