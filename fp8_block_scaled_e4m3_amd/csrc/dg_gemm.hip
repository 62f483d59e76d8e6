// dg_gemm.hip -- gfx950 kernels for the fine-grained-scaled FP8 E4M3 NT GEMM.
//
// What is computed ("DeepGEMM: clean and efficient FP8 GEMM kernels with
// fine-grained scaling", nipponese.news translation of the README, intro and
// usage paragraphs; scale granularity from DeepSeek-V3's fine-grained scheme):
//
//   D[m,n] = bf16( sum_kb sA[m,kb] * sB[n/128,kb] * sum_{k in kb} A[m,k] * B[n,k] )
//
// How it maps onto gfx950:
//  * One V_MFMA_F32_16X16X128_F8F6F4 (E4M3 x E4M3) covers exactly one 128-wide
//    K block of a 16x16 output sub-tile, so each K block's partial is produced
//    by a single MFMA with a zero accumulator and is promoted at once:
//    acc = fma(partial, sA*sB, acc) in fp32, K blocks ascending (the README's
//    two-level accumulation, done here on the VALU next to the matrix core).
//  * The MFMA's "M" side is fed with B rows and its "N" side with A rows, so a
//    lane's four results belong to one A row and four adjacent output columns:
//    one scale product sA[m]*sB[nb] serves four FMAs and sB is a wave-uniform
//    scalar for each 16-column sub-tile (16 divides 128, so a sub-tile never
//    straddles two B scale blocks even when BLOCK_N is not a power of two).
//  * Operand tiles (BLOCK_M + BLOCK_N rows of 128 K-bytes) go global -> LDS with
//    16-byte direct-to-LDS loads, two stages (one K block in flight while the
//    other is consumed), rows XOR-swizzled in 16-byte chunks so that the
//    MFMA-fragment reads are bank-conflict free.
//  * A persistent grid walks the tile list.  Tiles are handed out so that the
//    workgroups resident on one XCD (dispatch is round-robin over the 8 XCDs)
//    work on a compact block of the output and share A and B through that
//    XCD's L2.  Contiguous tiles look up their group in m_indices; masked tiles
//    are enumerated on the device from masked_m (the host never reads it), so
//    only row blocks that hold valid rows are visited.
//  * The epilogue converts to BF16 with the hardware RNE convert and stores
//    8 bytes per lane; padding rows (contiguous) and rows >= masked_m (masked)
//    are never written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKBlock = 128;        // K bytes per scale block == K of one MFMA
constexpr int kMaxMaskedGroups = 1024;
constexpr int kXcds = 8;

// 16-byte chunk swizzle of a 128-byte LDS row.  Depends on row bits 0..3 only,
// so it is a per-lane constant for fragment reads (rows 16q + lane%16); it makes
// 8 and 16 consecutive rows read at one logical chunk hit distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maximum.
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Copy 8 consecutive 128-byte rows into LDS (one wave instruction, 1 KB).
// `row_ptr` is this lane's source row; chunk = lane % 8 ^ swz(row).
__device__ __forceinline__ void dma_rows8(const uint8_t* row_ptr, int lrow8, int lane,
                                          uint8_t* lds_dst) {
    const int pc = lane & 7;
    const int lc = pc ^ swz(lrow8);
    __builtin_amdgcn_global_load_lds((const void*)(row_ptr + lc * 16), (lds_void*)lds_dst, 16, 0, 0);
}

template <int BM, int BN, int WM, int WN, int LAYOUT>
__global__ void __launch_bounds__(WM * WN * 64)
dg_gemm_kernel(const GemmParams p) {
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int ROWS = BM + BN;
    constexpr int STAGE = ROWS * kKBlock;
    constexpr int LOADS = ROWS / 8;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "block rows must be a multiple of 8");
    static_assert(WTN <= 128, "a wave's columns may touch at most two B scale blocks");

    __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGE];
    __shared__ int s_prefix[LAYOUT == kMasked ? kMaxMaskedGroups + 1 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int KB = p.kblocks;

    // ---- masked layout: valid row blocks per group, exclusive prefix in LDS ----
    int total_tiles = p.num_tiles;
    if constexpr (LAYOUT == kMasked) {
        const int G = p.num_groups;
        if (wave == 0) {
            const int per = (G + 63) / 64;
            int local = 0;
            for (int i = 0; i < per; ++i) {
                const int g = lane * per + i;
                if (g < G) {
                    int mm = p.masked_m[g];
                    mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
                    local += (mm + BM - 1) / BM;
                }
            }
            int incl = local;
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            int run = incl - local;
            for (int i = 0; i < per; ++i) {
                const int g = lane * per + i;
                if (g < G) {
                    s_prefix[g] = run;
                    int mm = p.masked_m[g];
                    mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
                    run += (mm + BM - 1) / BM;
                }
            }
            if (lane == 63) s_prefix[G] = incl;
        }
        __syncthreads();
        total_tiles = s_prefix[G] * p.tiles_n;
    }

    const int P = gridDim.x;
    const int w = blockIdx.x;
    for (int step = 0;; ++step) {
        // ---- tile index: XCD-aware hand-out of the linear tile order ----
        int L;
        if (p.xcd_remap) L = step * P + (w % kXcds) * (P / kXcds) + (w / kXcds);
        else L = step * P + w;
        if (step * P >= total_tiles) break;
        if (L >= total_tiles) continue;   // uniform; this workgroup idles this step

        int g = 0, mb, nb, valid_rows;
        if constexpr (LAYOUT == kMasked) {
            const int q = L / p.tiles_n;
            nb = L % p.tiles_n;
            int lo = 0, hi = p.num_groups;           // largest g with prefix[g] <= q
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_prefix[mid] <= q) lo = mid; else hi = mid;
            }
            g = lo;
            mb = q - s_prefix[g];
            int mm = p.masked_m[g];
            mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
            valid_rows = mm - mb * BM;
        } else {
            const int gsz = p.group_m * p.tiles_n;
            const int grp = L / gsz;
            const int first_m = grp * p.group_m;
            const int gm = min(p.tiles_m - first_m, p.group_m);
            const int r = L - grp * gsz;
            mb = first_m + r % gm;
            nb = r / gm;
            valid_rows = p.rows - mb * BM;
            if constexpr (LAYOUT == kContiguous) {
                g = p.m_indices[mb * BM];
                if (g < 0 || g >= p.num_groups) continue;   // padding block / no such group
            }
        }
        valid_rows = valid_rows > BM ? BM : valid_rows;
        const int m0 = mb * BM, n0 = nb * BN;

        const uint8_t* a_base = p.a + (LAYOUT == kMasked ? (long)g * p.a_gstride : 0);
        const float* sa_base = p.sa + (LAYOUT == kMasked ? (long)g * p.sa_gstride : 0);
        const uint8_t* b_base = p.b + (long)g * p.b_gstride;
        const float* sb_base = p.sb + (long)g * p.sb_gstride;
        uint16_t* d_base = p.d + (LAYOUT == kMasked ? (long)g * p.d_gstride : 0);
        const int a_last = p.rows - 1, b_last = p.n - 1;

        // ---- this lane's rows for the operand copies (clamped: tails read real rows) ----
        auto issue_stage = [&](uint8_t* smem, int kb) {
            for (int j = wave; j < LOADS; j += NW) {
                const int srow = j * 8 + (lane >> 3);
                const uint8_t* src;
                if (j * 8 < BM) {
                    int r = m0 + srow;
                    r = r > a_last ? a_last : r;
                    src = a_base + (long)r * p.lda + (long)kb * kKBlock;
                } else {
                    int r = n0 + srow - BM;
                    r = r > b_last ? b_last : r;
                    src = b_base + (long)r * p.ldb + (long)kb * kKBlock;
                }
                dma_rows8(src, srow, lane, smem + j * 1024);
            }
        };

        // ---- per-lane scale sources ----
        const float* sa_lane[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            int r = m0 + wm * WTM + fm * 16 + lrow;
            r = r > a_last ? a_last : r;
            sa_lane[fm] = sa_base + r;
        }
        const int wcol0 = n0 + wn * WTN;
        const int nb_lo = min(wcol0 / kKBlock, p.nblocks - 1);
        const int nb_hi = min(nb_lo + 1, p.nblocks - 1);
        unsigned hi_mask = 0;   // bit fn set: sub-tile fn uses nb_hi
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            if ((wcol0 + fn * 16) / kKBlock > nb_lo) hi_mask |= 1u << fn;
        const float* sb_lo_ptr = sb_base + (long)nb_lo * KB;
        const float* sb_hi_ptr = sb_base + (long)nb_hi * KB;
        const bool wave_active = wm * WTM < valid_rows;

        v4f acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = v4f{0.f, 0.f, 0.f, 0.f};

        // per-lane LDS byte offsets of the two 16-byte halves of a fragment row
        const int c0 = ((2 * lgrp) ^ swz(lrow)) * 16;
        const int c1 = ((2 * lgrp + 1) ^ swz(lrow)) * 16;

        struct Scales { float a[FM]; float bl, bh; };
        auto load_scales = [&](Scales& sc, int kb) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) sc.a[fm] = sa_lane[fm][(long)kb * p.ld_sa];
            sc.bl = sb_lo_ptr[kb];
            sc.bh = sb_hi_ptr[kb];
        };

        auto compute_stage = [&](const uint8_t* smem, const Scales& sc) {
            if (!wave_active) return;
            v8i af[FM];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const uint8_t* rowp = smem + (wm * WTM + fm * 16 + lrow) * kKBlock;
                const v4i lo = *(const v4i*)(rowp + c0);
                const v4i hi = *(const v4i*)(rowp + c1);
                af[fm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const uint8_t* rowp = smem + (BM + wn * WTN + fn * 16 + lrow) * kKBlock;
                const v4i lo = *(const v4i*)(rowp + c0);
                const v4i hi = *(const v4i*)(rowp + c1);
                const v8i bf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const float sbv = ((hi_mask >> fn) & 1u) ? sc.bh : sc.bl;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bf, af[fm], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    const float s = sc.a[fm] * sbv;
                    acc[fm][fn][0] = __builtin_fmaf(part[0], s, acc[fm][fn][0]);
                    acc[fm][fn][1] = __builtin_fmaf(part[1], s, acc[fm][fn][1]);
                    acc[fm][fn][2] = __builtin_fmaf(part[2], s, acc[fm][fn][2]);
                    acc[fm][fn][3] = __builtin_fmaf(part[3], s, acc[fm][fn][3]);
                }
            }
        };

        // ---- K loop: two LDS stages, loop unrolled by two so stage buffers are static.
        // The scales of K block kb+1 are fetched while block kb is consumed. ----
        Scales sc0, sc1;
        load_scales(sc0, 0);
        issue_stage(smem0, 0);
        for (int kb = 0; kb < KB; kb += 2) {
            wait_vmem_all();
            __syncthreads();
            if (kb + 1 < KB) {
                issue_stage(smem1, kb + 1);
                load_scales(sc1, kb + 1);
            }
            compute_stage(smem0, sc0);
            if (kb + 1 >= KB) break;
            wait_vmem_all();
            __syncthreads();
            if (kb + 2 < KB) {
                issue_stage(smem0, kb + 2);
                load_scales(sc0, kb + 2);
            }
            compute_stage(smem1, sc1);
        }

        // ---- epilogue: BF16 RNE, 8-byte stores, skip padding / masked / tail rows ----
        if (wave_active) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int lr = wm * WTM + fm * 16 + lrow;     // row inside the tile
                bool row_ok = lr < valid_rows;
                if constexpr (LAYOUT == kContiguous) {
                    if (row_ok) row_ok = p.m_indices[m0 + lr] >= 0;
                }
                if (!row_ok) continue;
                uint16_t* drow = d_base + (long)(m0 + lr) * p.ldd;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int col = wcol0 + fn * 16 + lgrp * 4;
                    if (col < p.n) {
                        v4bf o;
                        o.x = (__bf16)acc[fm][fn][0];
                        o.y = (__bf16)acc[fm][fn][1];
                        o.z = (__bf16)acc[fm][fn][2];
                        o.w = (__bf16)acc[fm][fn][3];
                        *(v4bf*)(drow + col) = o;
                    }
                }
            }
        }
        __syncthreads();   // every wave is done with both stages before the next tile
    }
}

template <int BM, int BN, int WM, int WN, int LAYOUT>
static hipError_t launch_cfg(const GemmParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, LAYOUT>), dim3(grid), dim3(WM * WN * 64), 0, s, p);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int LAYOUT>
static hipError_t occupancy_cfg(int* blocks) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks, reinterpret_cast<const void*>(&dg_gemm_kernel<BM, BN, WM, WN, LAYOUT>), WM * WN * 64, 0);
}

#define DG_CFG(ID, LAYOUT, BM, BN, WM, WN, EFF) \
    {ID, LAYOUT, BM, BN, WM, WN, EFF, &launch_cfg<BM, BN, WM, WN, LAYOUT>, &occupancy_cfg<BM, BN, WM, WN, LAYOUT>}

static const KernelConfig kConfigs[] = {
    // dense
    DG_CFG(0, kDense, 256, 224, 4, 2, 1.00),
    DG_CFG(1, kDense, 256, 256, 4, 2, 1.00),
    DG_CFG(2, kDense, 128, 128, 2, 2, 0.55),
    DG_CFG(3, kDense, 64, 112, 4, 1, 0.35),
    // contiguous (BLOCK_M = the 128-row segment alignment)
    DG_CFG(10, kContiguous, 128, 256, 2, 4, 1.00),
    DG_CFG(11, kContiguous, 128, 128, 2, 2, 0.55),
    // masked
    DG_CFG(20, kMasked, 256, 128, 4, 2, 1.00),
    DG_CFG(21, kMasked, 128, 128, 2, 2, 1.00),
};

const KernelConfig* kernel_configs(int* count) {
    *count = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
    return kConfigs;
}

}  // namespace dg
