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
    int wk;                // K groups of waves (1, or 2: each takes every other K block of a tile)
    double eff;            // relative throughput used by the planner
    bool all_formats;      // compiled for E5M2 operands too (else E4M3 only)
    bool shape_specialised;   // has instances for the shapes of kSpecShapes (N and K fixed at compile time)
    hipError_t (*launch)(const GemmParams&, int grid, hipStream_t);
    hipError_t (*occupancy)(int* blocks_per_cu);
};

// Shapes with their own compiled instances in the configurations marked
// shape_specialised (N and K/128 are compile-time constants there; every operand
// format the configuration runs):
// the DeepSeek-V3 projections of the workloads -- dense N = 7168 with K = 7168 (hidden
// width) or K = 2048 (expert width), grouped (contiguous and masked) N = 4096, K = 7168.
struct SpecShape {
    bool grouped;          // contiguous and masked layouts (else dense)
    int n, kblocks;
};
constexpr SpecShape kSpecShapes[] = {{false, 7168, 56}, {false, 7168, 16}, {true, 4096, 56}};
constexpr int kNumSpecShapes = sizeof(kSpecShapes) / sizeof(kSpecShapes[0]);

// The compiled tile configurations: X(id, layout, BLOCK_M, BLOCK_N, waves along M, waves
// along N, K groups (1, or 2: the K blocks of a tile split between two wave groups whose
// sums are added at the end), MFMA tile (16 or 32), LDS stages, relative throughput for
// the planner, pipelined variant fits the registers, E5M2 instances, shape instances).
// dg_gemm.hip instantiates a kernel for each row; the planner reads the same rows.
#define DG_CONFIG_TABLE(X)                                                   \
    /* dense */                                                              \
    X(0, kDense, 256, 224, 4, 2, 1, 16, 2, 1.00, false, false, false)       \
    X(1, kDense, 256, 224, 8, 1, 1, 32, 2, 0.90, false, false, false)       \
    X(2, kDense, 128, 128, 2, 2, 1, 16, 4, 0.55, false, false, false)       \
    X(3, kDense, 64, 112, 4, 1, 1, 16, 4, 0.35, false, true, true)          \
    X(4, kDense, 128, 224, 4, 2, 1, 16, 3, 0.80, true, false, false)        \
    X(5, kDense, 256, 256, 4, 2, 1, 16, 2, 1.15, true, true, true)          \
    X(6, kDense, 64, 64, 4, 1, 1, 16, 4, 0.32, false, true, false)          \
    X(7, kDense, 64, 64, 4, 1, 2, 16, 4, 0.35, false, true, false)          \
    /* contiguous (BLOCK_M = the 128-row segment alignment, or two of them) */ \
    X(10, kContiguous, 128, 256, 2, 4, 1, 16, 3, 1.00, false, false, false) \
    X(11, kContiguous, 128, 128, 2, 2, 1, 16, 4, 0.55, false, true, false)  \
    X(12, kContiguous, 128, 256, 2, 4, 1, 16, 2, 0.95, true, false, false)  \
    X(13, kContiguous, 256, 256, 4, 2, 1, 16, 2, 1.30, false, true, true)   \
    /* masked */                                                             \
    X(20, kMasked, 256, 128, 8, 1, 1, 16, 3, 1.00, false, false, false)     \
    X(21, kMasked, 128, 128, 2, 2, 1, 16, 4, 1.00, false, true, false)      \
    X(22, kMasked, 256, 128, 4, 2, 1, 16, 3, 0.90, false, false, false)     \
    X(23, kMasked, 128, 256, 2, 4, 1, 16, 3, 1.15, false, true, false)      \
    X(24, kMasked, 256, 256, 4, 2, 1, 16, 2, 1.10, false, true, true)

// Table of compiled configurations (defined in dg_gemm.hip).
const KernelConfig* kernel_configs(int* count);

// FP8 casts with fine-grained scales (defined in dg_quant.hip).
// q_e5m2: codes in E5M2 (scale amax / 57344) instead of E4M3 (amax / 448)
hipError_t launch_quant_1x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq, float* sa,
                              long ld_sa, int q_e5m2, hipStream_t stream);
hipError_t launch_quant_128x128(const void* x, int x_bf16, long ldx, int rows, int k, uint8_t* q, long ldq,
                                float* sb, int q_e5m2, hipStream_t stream);
// sA from row-major [groups][rows][ld_in] to MN-major [groups][kblocks][ld_sa] (dg_quant.hip).
hipError_t launch_sa_mn_major(const float* in, long ld_in, float* out, long ld_sa, int rows, int kblocks, int groups,
                              hipStream_t stream);

}  // namespace dg
