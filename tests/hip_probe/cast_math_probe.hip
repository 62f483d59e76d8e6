// cast_math_probe.hip -- test probe (not part of libdg.so): runs the FP8 casts' own
// device arithmetic (dg_cast_math.h, the header the cast kernels include) over large
// input sets on the GPU and counts where it differs from the IEEE single-precision
// division, bit for bit.
//
//   probe_rcp_exact: rcp_exact(s) against 1/s for every fp32 bit pattern in [lo, hi]
//                    (raw != 0: the hardware reciprocal estimate alone, which must
//                    differ somewhere -- evidence that the comparison can fail).
//   probe_div_fast : div_fast(x, s, rcp_exact(s)) against x/s for given scales s and,
//                    per scale, the values x = RN(t * s) and their fp32 neighbours for
//                    every multiplier t in a table (the FP8 formats' values and rounding
//                    ties), plus pseudo-random x in [-FMAX*s, FMAX*s].
// Both host functions allocate their own device counters, launch, wait and copy the
// counts back; they return 0 or a HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../fp8_block_scaled_e4m3_amd/csrc/dg_cast_math.h"

using namespace dg::castmath;

namespace {

__device__ void record(unsigned long long local, uint32_t first, unsigned long long* bad, uint32_t* first_bad) {
    if (local) {
        atomicAdd(bad, local);
        atomicMin(first_bad, first);
    }
}

__global__ void __launch_bounds__(256) rcp_kernel(uint32_t lo, uint32_t count, int raw, unsigned long long* bad,
                                                  uint32_t* first_bad) {
    unsigned long long local = 0;
    uint32_t first = 0xFFFFFFFFu;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const uint32_t bits = lo + i;
        const float s = __uint_as_float(bits);
        const float a = raw ? __builtin_amdgcn_rcpf(s) : rcp_exact(s);
        const float b = __fdiv_rn(1.0f, s);
        if (__float_as_uint(a) != __float_as_uint(b)) {
            ++local;
            first = bits < first ? bits : first;
        }
        if (stride > 0xFFFFFFFFu - i) break;   // i + stride would wrap
    }
    record(local, first, bad, first_bad);
}

// counter-based pseudo-random 32-bit value (a 32-bit integer hash, Wellons' "lowbias32")
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// one workgroup per scale; its threads walk the x values of that scale
__global__ void __launch_bounds__(256) div_kernel(const float* scales, const float* mult, int nmult, int nrand,
                                                  float fmax, unsigned long long* bad, uint32_t* first_bad) {
    const float s = scales[blockIdx.x];
    const float r = rcp_exact(s);
    const int n = 3 * nmult + nrand;
    unsigned long long local = 0;
    uint32_t first = 0xFFFFFFFFu;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        float x;
        if (i < 3 * nmult) {
            const float x0 = mult[i / 3] * s;                  // RN(t * s)
            const int off = i % 3;                             // itself, one ulp down, one ulp up
            x = off == 0 ? x0 : __uint_as_float(__float_as_uint(x0) + (off == 1 ? -1 : 1));
            if (x0 == 0.f) x = x0;
        } else {
            const uint32_t h = hash32((uint32_t)i * 2654435761u ^ blockIdx.x * 40503u);
            const float u = (float)(h >> 8) * 0x1p-24f;          // [0, 1)
            x = (h & 1u ? -1.f : 1.f) * u * fmax * s;
        }
        const float a = div_fast(x, s, r);
        const float b = __fdiv_rn(x, s);
        if (__float_as_uint(a) != __float_as_uint(b)) {
            ++local;
            first = blockIdx.x < first ? blockIdx.x : first;
        }
    }
    record(local, first, bad, first_bad);
}

int run(void (*launch)(unsigned long long*, uint32_t*), unsigned long long* bad_out, uint32_t* first_out) {
    unsigned long long* d_bad = nullptr;
    uint32_t* d_first = nullptr;
    hipError_t e = hipMalloc(&d_bad, sizeof(*d_bad));
    if (e == hipSuccess) e = hipMalloc(&d_first, sizeof(*d_first));
    if (e == hipSuccess) e = hipMemset(d_bad, 0, sizeof(*d_bad));
    if (e == hipSuccess) e = hipMemset(d_first, 0xFF, sizeof(*d_first));
    if (e == hipSuccess) {
        launch(d_bad, d_first);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(bad_out, d_bad, sizeof(*d_bad), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(first_out, d_first, sizeof(*d_first), hipMemcpyDeviceToHost);
    if (d_bad) (void)hipFree(d_bad);
    if (d_first) (void)hipFree(d_first);
    return (int)e;
}

uint32_t g_lo, g_count;
int g_raw;
const float *g_scales, *g_mult;
int g_ns, g_nm, g_nr;
float g_fmax;

}  // namespace

extern "C" int probe_rcp_exact(uint32_t lo, uint32_t hi, int raw, unsigned long long* bad, uint32_t* first_bad) {
    if (hi < lo) return -1;
    g_lo = lo;
    g_raw = raw;
    g_count = hi - lo + 1;   // hi - lo < 2^32 - 1 for every range used
    return run(
        [](unsigned long long* b, uint32_t* f) {
            hipLaunchKernelGGL(rcp_kernel, dim3(256 * 64), dim3(256), 0, nullptr, g_lo, g_count, g_raw, b, f);
        },
        bad, first_bad);
}

// scales, mult: HOST arrays (copied to the device here); first_bad receives the index of
// the first scale with a mismatch
extern "C" int probe_div_fast(const float* scales, int nscales, const float* mult, int nmult, int nrand, float fmax,
                              unsigned long long* bad, uint32_t* first_bad) {
    if (nscales <= 0 || nmult < 0 || nrand < 0) return -1;
    float *d_s = nullptr, *d_m = nullptr;
    hipError_t e = hipMalloc(&d_s, sizeof(float) * nscales);
    if (e == hipSuccess) e = hipMalloc(&d_m, sizeof(float) * (nmult > 0 ? nmult : 1));
    if (e == hipSuccess) e = hipMemcpy(d_s, scales, sizeof(float) * nscales, hipMemcpyHostToDevice);
    if (e == hipSuccess && nmult > 0) e = hipMemcpy(d_m, mult, sizeof(float) * nmult, hipMemcpyHostToDevice);
    int rc = (int)e;
    if (e == hipSuccess) {
        g_scales = d_s;
        g_mult = d_m;
        g_ns = nscales;
        g_nm = nmult;
        g_nr = nrand;
        g_fmax = fmax;
        rc = run(
            [](unsigned long long* b, uint32_t* f) {
                hipLaunchKernelGGL(div_kernel, dim3(g_ns), dim3(256), 0, nullptr, g_scales, g_mult, g_nm, g_nr,
                                   g_fmax, b, f);
            },
            bad, first_bad);
    }
    if (d_s) (void)hipFree(d_s);
    if (d_m) (void)hipFree(d_m);
    return rc;
}
