// dg_internal.h -- shared between the host dispatcher (dg_api.cpp) and the
// kernel translation unit (dg_gemm.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

// Every pointer is a device pointer.  Strides are in elements of the pointee.
struct GemmParams {
    const uint8_t* a;      long lda;  long a_gstride;    // masked: bytes between groups
    const float* sa;       long ld_sa; long sa_gstride;  // masked: floats between groups
    const uint8_t* b;      long ldb;  long b_gstride;    // grouped: bytes between groups
    const float* sb;       long sb_gstride;              // grouped: floats between groups
    uint16_t* d;           long ldd;  long d_gstride;    // masked: elements between groups
    const int* m_indices;  // contiguous
    const int* masked_m;   // masked
    int rows;              // dense: M; contiguous: m_total; masked: max_m
    int n, k;
    int kblocks, nblocks;  // K/128, ceil(N/128)
    int num_groups;
    int tiles_m, tiles_n;  // tile grid (masked: per group)
    int num_tiles;         // dense/contiguous: exact; masked: upper bound
    int group_m;           // raster: tiles_m rows visited together
    int xcd_remap;         // 1 when the grid is a multiple of the XCD count
    int fmt;               // operand formats: bit 0 set = A is E5M2, bit 1 set = B is E5M2 (else E4M3)
};

struct KernelConfig {
    int id;
    int layout;
    int bm, bn, wm, wn;
    double eff;            // relative throughput used by the planner
    bool all_formats;      // compiled for E5M2 operands too (else E4M3 only)
    bool k_specialised;    // has instances with K/128 fixed at compile time (kSpecKBlocks)
    hipError_t (*launch)(const GemmParams&, int grid, hipStream_t);
    hipError_t (*occupancy)(int* blocks_per_cu);
};

// K/128 values with their own compiled instances (every operand format the configuration
// runs) in the configurations marked k_specialised: K = 7168 and K = 2048, the hidden and expert widths of the
// DeepSeek-V3 shapes the workloads use.
constexpr int kSpecKBlocks[2] = {56, 16};

// Table of compiled configurations (defined in dg_gemm.hip).
const KernelConfig* kernel_configs(int* count);

// FP8 casts with fine-grained scales (defined in dg_quant.hip).
// q_e5m2: codes in E5M2 (scale amax / 57344) instead of E4M3 (amax / 448)
hipError_t launch_quant_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                              long ld_sa, int q_e5m2, hipStream_t stream);
hipError_t launch_quant_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq,
                                float* sb, int q_e5m2, hipStream_t stream);

}  // namespace dg
