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
// Both quotients are the correctly rounded fp32 ones (what an IEEE division gives;
// dg_cast_math.h reaches them without one on the fast path), so the codes are a
// deterministic function of the input.  Each kernel reads its input once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_cast_math.h"
#include "dg_internal.h"

namespace dg {

namespace {

using namespace castmath;

constexpr int kQBlock = 128;

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);   // bf16 -> fp32 is exact
}

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

// Maximum over each aligned group of L lanes (L = 16 or 32) of non-negative, non-NaN
// values, through the cross-lane paths of the vector ALU rather than LDS: DPP lane
// swaps within quads (lanes 1 and 2 apart), mirrors within 8- and 16-lane rows, and
// for L = 32 the swap of adjacent 16-lane rows.  Each step combines every lane with a
// lane of the other half of its current span, so after log2(L) steps every lane of a
// group holds the group's maximum.  Non-negative floats (+0 to +inf) order like their
// bit patterns read as signed integers, so the steps take integer maxima.
template <int CTRL>
__device__ __forceinline__ int dpp_max_bits(int x) {
    const int o = __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
    return o > x ? o : x;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
    static_assert(L == 16 || L == 32, "group of 16 or 32 lanes");
    int b = __builtin_bit_cast(int, v);
    b = dpp_max_bits<0xB1>(b);    // quad_perm [1,0,3,2]
    b = dpp_max_bits<0x4E>(b);    // quad_perm [2,3,0,1]
    b = dpp_max_bits<0x141>(b);   // row_half_mirror
    b = dpp_max_bits<0x140>(b);   // row_mirror
    if constexpr (L == 32) {
        const auto sw = __builtin_amdgcn_permlane16_swap((unsigned)b, (unsigned)b, false, false);
        const int lo = (int)sw[0], hi = (int)sw[1];
        b = lo > hi ? lo : hi;
    }
    return __builtin_bit_cast(float, b);
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
// A thread handles kRowsPerThread row blocks, their loads all in flight before any
// is reduced.  Blocks are numbered K block fastest, so a workgroup reads long
// contiguous stretches of each row.  RUN (when kRowsPerThread divides K/128): a
// thread's blocks are consecutive K blocks of one row, so one row split and one
// address serve all of them (the split and the 64-bit addressing are a large share
// of this kernel's vector instructions); otherwise they are GPW blocks apart and each
// finds its own row.
constexpr int kRowsPerThread = 4;

template <typename T, int FMT, bool RUN>
__global__ void __launch_bounds__(256)
quant_1x128_kernel(const T* __restrict__ x, long ldx, int rows, int kblocks, DivU32 kdiv, uint8_t* __restrict__ q,
                   long ldq, float* __restrict__ sa, long ld_sa) {
    constexpr int N = Vec<T>::N, L = kQBlock / N, GPW = 256 / L;   // groups of L lanes per workgroup
    constexpr int R = kRowsPerThread;
    const int lg = threadIdx.x % L, grp = threadIdx.x / L;
    // (the host keeps rows * kblocks below 2^31)
    const unsigned groups_total = (unsigned)rows * (unsigned)kblocks;
    float v[R][N];
    if constexpr (RUN) {
        // run G = blocks [G*R, G*R + R) of one row; kdiv divides by kblocks / R
        const unsigned G = blockIdx.x * (unsigned)GPW + grp;
        if (G * R >= groups_total) return;              // uniform over the L lanes of a group
        const unsigned row = div_u32(G, kdiv), kb0 = (G - row * (unsigned)(kblocks / R)) * R;
        const T* xb = x + (long)row * ldx + kb0 * kQBlock + lg * N;
#pragma unroll
        for (int r = 0; r < R; ++r) Vec<T>::load(xb + r * kQBlock, v[r]);
        uint8_t* qb = q + (long)row * ldq + kb0 * kQBlock + lg * N;
        float* sb = sa + (long)kb0 * ld_sa + row;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float amax = group_max<L>(amax_of(v[r], N, 0.f));
            const float scale = block_scale<FMT>(amax);
            const bool fast = wave_all(fast_scale(scale) && !any_nan(v[r], N));
            store_codes<N, FMT>(qb + r * kQBlock, v[r], scale, fast);
            if (lg == 0) sb[r * ld_sa] = scale;
        }
    } else {
        // workgroup w handles groups [w*GPW*R, (w+1)*GPW*R); group g = (row, kb)
        const unsigned g0 = blockIdx.x * (unsigned)(GPW * R) + grp;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const unsigned g = g0 + r * GPW;
            if (g < groups_total) {
                const unsigned row = div_u32(g, kdiv), kb = g - row * (unsigned)kblocks;
                Vec<T>::load(x + (long)row * ldx + kb * kQBlock + lg * N, v[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const unsigned g = g0 + r * GPW;
            if (g >= groups_total) break;                   // uniform over the L lanes of a group
            const float amax = group_max<L>(amax_of(v[r], N, 0.f));
            const float scale = block_scale<FMT>(amax);
            const unsigned row = div_u32(g, kdiv), kb = g - row * (unsigned)kblocks;
            const bool fast = wave_all(fast_scale(scale) && !any_nan(v[r], N));
            store_codes<N, FMT>(q + (long)row * ldq + kb * kQBlock + lg * N, v[r], scale, fast);
            if (lg == 0) sa[(long)kb * ld_sa + row] = scale;
        }
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

// sA layout transform: per-row scales stored row-major, in[g][row][kb] (row stride
// ld_in), to the MN-major layout the GEMMs read, out[g][kb][row] (row stride ld_sa) --
// the README's utility that returns the LHS scales column-major with an aligned leading
// dimension.  A 32 x 32 tile goes through LDS so that both the reads (along kb) and the
// writes (along rows) are contiguous; the padding columns [rows, ld_sa) are not written.
constexpr int kTT = 32;

__global__ void __launch_bounds__(256)
sa_mn_major_kernel(const float* __restrict__ in, long ld_in, float* __restrict__ out, long ld_sa, int rows,
                   int kblocks) {
    __shared__ float tile[kTT][kTT + 1];
    const int r0 = blockIdx.x * kTT, k0 = blockIdx.y * kTT, g = blockIdx.z;
    const float* src = in + (long)g * rows * ld_in;
    float* dst = out + (long)g * kblocks * ld_sa;
    const int tx = threadIdx.x % kTT, ty = threadIdx.x / kTT;   // 32 x 8 threads
#pragma unroll
    for (int i = 0; i < kTT; i += 8) {
        const int r = r0 + ty + i, k = k0 + tx;
        if (r < rows && k < kblocks) tile[ty + i][tx] = src[(long)r * ld_in + k];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTT; i += 8) {
        const int k = k0 + ty + i, r = r0 + tx;
        if (r < rows && k < kblocks) dst[(long)k * ld_sa + r] = tile[tx][ty + i];
    }
}

}  // namespace

namespace {

template <int FMT>
hipError_t launch_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                        long ld_sa, hipStream_t stream) {
    const int kblocks = k / kQBlock;
    const bool run = kblocks % kRowsPerThread == 0;
    const DivU32 kdiv = make_div_u32((uint32_t)(run ? kblocks / kRowsPerThread : kblocks));
    const long per_wg = (x_bf16 ? 256 / 16 : 256 / 32) * (long)kRowsPerThread;   // groups per workgroup
    // row chunks small enough for 32-bit group indices inside the kernel
    const long chunk = ((1l << 30) / kblocks) > 0 ? ((1l << 30) / kblocks) : 1;
    for (long r0 = 0; r0 < rows; r0 += chunk) {
        const int nr = (int)(rows - r0 < chunk ? rows - r0 : chunk);
        const long blocks = ((long)nr * kblocks + per_wg - 1) / per_wg;
        const uint16_t* xh = static_cast<const uint16_t*>(x) + r0 * ldx;
        const float* xf = static_cast<const float*>(x) + r0 * ldx;
        const dim3 grid((unsigned)blocks);
        if (x_bf16 && run)
            hipLaunchKernelGGL((quant_1x128_kernel<uint16_t, FMT, true>), grid, dim3(256), 0, stream, xh, ldx, nr,
                               kblocks, kdiv, q + r0 * ldq, ldq, sa + r0, ld_sa);
        else if (x_bf16)
            hipLaunchKernelGGL((quant_1x128_kernel<uint16_t, FMT, false>), grid, dim3(256), 0, stream, xh, ldx, nr,
                               kblocks, kdiv, q + r0 * ldq, ldq, sa + r0, ld_sa);
        else if (run)
            hipLaunchKernelGGL((quant_1x128_kernel<float, FMT, true>), grid, dim3(256), 0, stream, xf, ldx, nr,
                               kblocks, kdiv, q + r0 * ldq, ldq, sa + r0, ld_sa);
        else
            hipLaunchKernelGGL((quant_1x128_kernel<float, FMT, false>), grid, dim3(256), 0, stream, xf, ldx, nr,
                               kblocks, kdiv, q + r0 * ldq, ldq, sa + r0, ld_sa);
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

hipError_t launch_sa_mn_major(const float* in, long ld_in, float* out, long ld_sa, int rows, int kblocks, int groups,
                              hipStream_t stream) {
    const dim3 grid((unsigned)((rows + kTT - 1) / kTT), (unsigned)((kblocks + kTT - 1) / kTT), (unsigned)groups);
    hipLaunchKernelGGL(sa_mn_major_kernel, grid, dim3(256), 0, stream, in, ld_in, out, ld_sa, rows, kblocks);
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq,
                                float* sb, int q_e5m2, hipStream_t stream) {
    return q_e5m2 ? launch_128x128<1>(x, x_bf16, ldx, rows, k, q, ldq, sb, stream)
                  : launch_128x128<0>(x, x_bf16, ldx, rows, k, q, ldq, sb, stream);
}

}  // namespace dg
