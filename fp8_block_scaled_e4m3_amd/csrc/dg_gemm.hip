// dg_gemm.hip -- gfx950 kernels for the fine-grained-scaled FP8 E4M3 NT GEMM.
//
// What is computed ("DeepGEMM: clean and efficient FP8 GEMM kernels with
// fine-grained scaling", nipponese.news translation of the README, intro and
// usage paragraphs; scale granularity from DeepSeek-V3's fine-grained scheme):
//
//   D[m,n] = bf16( sum_kb sA[m,kb] * sB[n/128,kb] * sum_{k in kb} A[m,k] * B[n,k] )
//
// How it maps onto gfx950:
//  * One V_MFMA_F32_16X16X128_F8F6F4 (E4M3 x E4M3; either operand E5M2 through
//    the instruction's format fields, FMT below) covers exactly one 128-wide
//    K block of a 16x16 output sub-tile, so each K block's partial is produced
//    by a single MFMA with a zero accumulator and is promoted at once:
//    acc = fma(partial, sA*sB, acc) in fp32, K blocks ascending (the README's
//    two-level accumulation, done here on the VALU next to the matrix core).
//  * The MFMA's "M" side is fed with B rows and its "N" side with A rows, so a
//    lane's four results belong to one A row and four adjacent output columns:
//    one scale product sA[m]*sB[nb] serves four FMAs and sB is a wave-uniform
//    scalar for each 16-column sub-tile (16 divides 128, so a sub-tile never
//    straddles two B scale blocks even when BLOCK_N is not a power of two).
//  * Operand tiles (BLOCK_M + BLOCK_N rows of 128 K-bytes) and the tile's A
//    scales go global -> LDS with direct-to-LDS buffer loads into 2..4 stages (the
//    copies of a K block are issued as soon as the stage it reuses is free), rows
//    XOR-swizzled in 16-byte chunks so that the MFMA-fragment reads are bank-
//    conflict free.  B scales are wave-uniform scalar loads.
//  * A persistent grid walks the tile list.  Tiles are handed out so that the
//    workgroups resident on one XCD (dispatch is round-robin over the 8 XCDs)
//    work on a compact block of the output and share A and B through that
//    XCD's L2.  Contiguous tiles look up their group in m_indices; masked tiles
//    are enumerated on the device from masked_m (the host never reads it), so
//    only row blocks that hold valid rows are visited.
//  * The epilogue converts to BF16 with the hardware RNE convert; lane-group
//    swaps give each lane eight adjacent columns, stored 16 bytes at a time.
//    Padding rows (contiguous) and rows >= masked_m (masked) are never written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.h"

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const float lds_f32;

constexpr int kKBlock = 128;        // K bytes per scale block == K of one MFMA
constexpr int kMaxMaskedGroups = 1024;
constexpr int kXcds = 8;
constexpr int kMAlign = 128;        // contiguous layout: rows per segment block (alignment)

// 16-byte chunk swizzle of a 128-byte LDS row.  Depends on row bits 0..3 only,
// so it is a per-lane constant for fragment reads (rows 16q + lane%16); it makes
// 8 and 16 consecutive rows read at one logical chunk hit distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Raw buffer descriptor over `bytes` bytes from `base` (clamped to 4 GiB - 1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
    const unsigned n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFl ? 0xFFFFFFFFu : (unsigned)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

// Cache-policy bit of a buffer load: non-temporal (the lines are inserted for early
// eviction from L2; for data that no other workgroup will read again).
constexpr int kCpolNT = 2;

// One 16-byte-per-lane copy from a buffer straight into LDS (a named device
// function, so that only the device compilation ever checks the 16-byte form),
// with cache policy CPOL.
template <int CPOL = 0>
__device__ __forceinline__ void buffer_copy_lds16(__amdgpu_buffer_rsrc_t rs, lds_void* dst, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, soff, 0, CPOL);
}

// Workgroup barrier without a memory fence.  __syncthreads() also fences, which
// drains every outstanding load of the wave, including the copies of younger
// stages that should stay in flight; the callers wait for exactly what they need
// (wait_vmem_le) first.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maximum: at most N of
// this wave's vector memory loads may still be outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Lambdas of the kernel are always inlined: a call that stays out of line would put
// the accumulator arrays it captures by reference into scratch memory.
#define DG_INLINE __attribute__((always_inline))

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time (kernels and the
// host-side instance selection).
template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// MF selects the matrix instruction: 16 -> V_MFMA_F32_16X16X128_F8F6F4 (one
// instruction per 128-K block of a 16x16 sub-tile), 32 -> V_MFMA_F32_32X32X64_F8F6F4
// (two instructions per 128-K block of a 32x32 sub-tile; the second accumulates
// onto the first, so the promoted quantity is still the whole block's partial).
// The 32x32 form needs one scale product per 16 promotion FMAs instead of per 4,
// and its 32-column sub-tiles never straddle a 128-column scale block when the
// tile offsets are multiples of 32.
// FMT: operand formats, bit 0 = A is E5M2, bit 1 = B is E5M2 (else E4M3).  The
// matrix instruction's format fields take them directly (B rows feed the
// instruction's first operand, A rows its second).
// NC, KC > 0: an instance for N == NC and K/128 == KC only (tile counts, scale-row
// offsets, the column guard, loop trip counts and the split into stage groups are
// then compile-time constants); 0: any N, K.
// WK = 2 (dense layout, per-tile loop): the workgroup holds two K groups of WM x WN
// waves.  Group wk computes the whole tile over the K blocks kb with kb % 2 == wk
// (each with its own promotion chain, K blocks ascending), so a tile's K loop takes
// half as many block steps, each step carrying one block per group; at the end of
// the tile group 0 adds group 1's fp32 sums to its own and stores the tile.  For
// small-M shapes with long K whose tiles leave CUs idle: there a tile's time is its
// chain of block steps, not the CU's share of the operand bytes.
template <int BM, int BN, int WM, int WN, int LAYOUT, int MF, int NST, bool PIPE, int FMT, int NC, int KC, int WK>
__global__ void __launch_bounds__(WM * WN * WK * 64)
dg_gemm_kernel(const GemmParams p, const uint8_t* __restrict__ a_ptr, const float* __restrict__ sa_ptr,
               const uint8_t* __restrict__ b_ptr, const float* __restrict__ sb_ptr, uint16_t* __restrict__ d_ptr) {
    constexpr int NWG = WM * WN;                   // waves of one K group
    constexpr int NW = NWG * WK;
    static_assert(WK == 1 || WK == 2, "one or two K groups");
    static_assert(WK == 1 || (LAYOUT == kDense && !PIPE), "K groups: dense layout, per-tile loop");
    constexpr int WTM = BM / WM, WTN = BN / WN;
    // operand formats (FMT bit 0: A is E5M2, bit 1: B is E5M2); the MFMA's first
    // source carries B rows and its second A rows.  Field values: 0 = E4M3, 1 = E5M2
    constexpr int FMT_SRC0 = (FMT >> 1) & 1, FMT_SRC1 = FMT & 1;
    constexpr int FM = WTM / MF, FN = WTN / MF;
    constexpr int NACC = MF * MF / 64;             // accumulator floats per lane per sub-tile
    constexpr int ROWS = BM + BN;
    // a stage holds the operand rows of one K block per K group (SUB bytes each) and,
    // behind them, each wave's copy of the A scales of its rows (64 fp32 values per wave)
    constexpr int SUB = ROWS * kKBlock;
    constexpr int STAGE = WK * SUB + NW * 256;
    constexpr int A_SLOTS = BM / 8, B_SLOTS = BN / 8;
    constexpr int A_PER = (A_SLOTS + NWG - 1) / NWG, B_PER = (B_SLOTS + NWG - 1) / NWG;
    static_assert(MF == 16 || MF == 32, "matrix instruction shape");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA tile");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "block rows must be a multiple of 8");
    static_assert(WTN <= 256, "a wave's columns touch at most three B scale blocks");
    static_assert(MF != 16 || WTN <= 128, "16-wide sub-tiles: a wave's columns touch at most two B scale blocks");
    static_assert(WTM <= 64, "one 4-byte-per-lane copy carries a wave's A scales");
    typedef float vacc __attribute__((ext_vector_type(NACC)));

    // NST stage buffers, each its own array so the compiler can prove that fragment
    // reads of one stage never alias the copies in flight into another.
    static_assert(NST >= 2 && NST <= 8, "2..8 LDS stages");
    __shared__ __attribute__((aligned(1024))) uint8_t smem0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t smem2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smem3[NST > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smem4[NST > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smem5[NST > 5 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smem6[NST > 6 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smem7[NST > 7 ? STAGE : 16];
    __shared__ int s_prefix[LAYOUT == kMasked ? kMaxMaskedGroups + 1 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = WK == 1 ? 0 : wave / NWG;        // K group
    const int wg = WK == 1 ? wave : wave % NWG;     // wave inside its K group
    const int wm = wg % WM, wn = wg / WM;
    const int lsub = lane & (MF - 1);             // row of the sub-tile this lane feeds / owns
    const int lgrp = lane / MF;                   // K group of the lane inside an operand fragment
    const int KBT = KC > 0 ? KC : p.kblocks;           // K blocks of the problem
    const int KB = (KBT + WK - 1) / WK;                // block steps of a tile's K loop
    static_assert((NC > 0) == (KC > 0), "shape instances fix N and K together");
    const int NN = NC > 0 ? NC : p.n;
    const int TILES_N = NC > 0 ? (NC + BN - 1) / BN : p.tiles_n;
    const int NBLK = NC > 0 ? (NC + kKBlock - 1) / kKBlock : p.nblocks;
    constexpr bool WHOLE_N = NC > 0 && NC % BN == 0;   // no tile has columns past N

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
        total_tiles = s_prefix[G] * TILES_N;
    }

    const int P = gridDim.x;
    const int w = blockIdx.x;
    constexpr int NSLOT = A_PER + B_PER;

    // ---- operand copies: 8-row slots dealt round robin to the waves.  Each lane's
    // 32-bit source offset inside a tile is the same for every tile and K block;
    // rows past an operand's end fall outside the tile's buffer descriptor, so their
    // copies read nothing and write zeros (their outputs are never stored). ----
    uint32_t a_off[A_PER], b_off[B_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int srow = min(wg + i * NWG, A_SLOTS - 1) * 8 + (lane >> 3);
        a_off[i] = (uint32_t)srow * (uint32_t)p.lda + (uint32_t)((((lane & 7) ^ swz(srow))) * 16);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int srow = min(wg + i * NWG, B_SLOTS - 1) * 8 + (lane >> 3);
        b_off[i] = (uint32_t)srow * (uint32_t)p.ldb + (uint32_t)((((lane & 7) ^ swz(BM + srow))) * 16);
    }
    // A scales: a wave's rows of a K block are contiguous in sA (MN-major), so they
    // travel to LDS with the block's operands, one 4-byte copy per lane (row
    // wm*WTM + lane) into the wave's own 256-byte area of the stage.  The K offset
    // is in the per-lane offset, which the descriptor bounds (rows past the end of
    // sA read zeros).
    const uint32_t sa_voff = (uint32_t)(wm * WTM + lane) * 4u;
    const int sa_lds = WK * SUB + wave * 256 + lsub * 4;   // this lane's row, sub-tile 0
    // B scale rows a wave reads per K block: MF=16 sub-tiles need at most two (the
    // wave's columns span at most 128); a 128-column wave tile at a multiple of 128
    // needs exactly one, so all of its sub-tiles share one scale product per row
    constexpr bool ONE_SB = MF == 16 && WTN == kKBlock && BN % kKBlock == 0;
    constexpr int NSB = MF == 16 ? (ONE_SB ? 1 : 2) : FN;

    // ---- one tile (or one pass of a two-group contiguous tile): everything its
    // copies, scales and epilogue need, all wave-uniform ----
    // (rows [row_lo, row_hi) of the tile are this pass's valid rows)
    struct Tile {
        int m0, row_lo, row_hi, wcol0, grp;
        unsigned hi_mask;
        int sb_off[NSB];
        bool active;
        __amdgpu_buffer_rsrc_t rs_a, rs_b, rs_sa;
        const float* sb_grp;
        uint16_t* d_tile;
    };
    // the tile hand-out: step s gives workgroup w the tile L(s, w); a contiguous
    // tile holding two groups yields two passes
    int step = 0, pass = 0, npass = 0, st_m0 = 0, st_n0 = 0, st_vr = 0;
    int pg[2] = {0, 0}, plo[2] = {0, 0}, phi[2] = {BM, BM};
    auto fetch_step = [&]() DG_INLINE -> bool {   // from `step` on, the first step with work
        for (;; ++step) {
            if (step * P >= total_tiles) return false;
            // ---- tile index: XCD-aware hand-out of the linear tile order ----
            int L;
            if (p.xcd_remap) {
                // Each XCD takes a contiguous share of the step's tiles.  Dense: a
                // partial last round is spread evenly over all eight XCDs rather than
                // filling the first ones (4-14% faster on 256x256 tiles with 24..248
                // tiles left; the grouped layouts measured slower with it).
                const int R = total_tiles - step * P;
                if (LAYOUT == kDense && R < P) {
                    const int per = (R + kXcds - 1) / kXcds;
                    const int j = (w % kXcds) * per + (w / kXcds);
                    if (w / kXcds >= per || j >= R) continue;   // uniform; idle this step
                    L = step * P + j;
                } else {
                    L = step * P + (w % kXcds) * (P / kXcds) + (w / kXcds);
                }
            } else {
                L = step * P + w;
            }
            if (L >= total_tiles) continue;   // uniform; this workgroup idles this step
            int g = 0, mb, nb, valid_rows;
            if constexpr (LAYOUT == kMasked) {
                // group g owns tiles [prefix[g], prefix[g+1]) * tiles_n, ordered N block
                // major and row block minor, so the row blocks sharing one B tile are
                // neighbours in the hand-out (same XCD, same step: B comes from L2 once)
                const int q = L / TILES_N;
                int lo = 0, hi = p.num_groups;           // largest g with prefix[g] <= q
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_prefix[mid] <= q) lo = mid; else hi = mid;
                }
                g = lo;
                const int vb = s_prefix[g + 1] - s_prefix[g];
                const int t = L - s_prefix[g] * TILES_N;
                nb = t / vb;
                mb = t - nb * vb;
                int mm = p.masked_m[g];
                mm = mm < 0 ? 0 : (mm > p.rows ? p.rows : mm);
                valid_rows = mm - mb * BM;
            } else {
                const int gsz = p.group_m * TILES_N;
                const int grp = L / gsz;
                const int first_m = grp * p.group_m;
                const int gm = min(p.tiles_m - first_m, p.group_m);
                const int r = L - grp * gsz;
                mb = first_m + r % gm;
                nb = r / gm;
                valid_rows = p.rows - mb * BM;
            }
            valid_rows = valid_rows > BM ? BM : valid_rows;
            st_m0 = mb * BM;
            st_n0 = nb * BN;
            st_vr = valid_rows;
            npass = 1;
            pg[0] = pg[1] = g;
            plo[0] = plo[1] = 0;
            phi[0] = phi[1] = BM;
            // Contiguous layout: the group of every 128-row segment block is the index
            // of its first row (-1 or out of range: padding, skipped).  A tile of two
            // segment blocks that belong to different groups is computed in two passes,
            // one per group, each keeping only its own rows.
            if constexpr (LAYOUT == kContiguous) {
                auto group_at = [&](int r) DG_INLINE {
                    if (r >= valid_rows) return -1;
                    const int v = p.m_indices[st_m0 + r];
                    return (v < 0 || v >= p.num_groups) ? -1 : v;
                };
                if constexpr (BM > kMAlign) {
                    static_assert(BM == 2 * kMAlign, "at most two segment blocks per tile");
                    const int g0 = group_at(0), g1 = group_at(kMAlign);
                    if (g0 < 0 && g1 < 0) continue;
                    if (g0 >= 0 && g1 == g0) {
                        pg[0] = g0;
                    } else if (g0 >= 0 && g1 < 0) {
                        pg[0] = g0;
                        phi[0] = kMAlign;
                    } else if (g0 < 0) {
                        pg[0] = g1;
                        plo[0] = kMAlign;
                    } else {
                        npass = 2;
                        pg[0] = g0;
                        phi[0] = kMAlign;
                        pg[1] = g1;
                        plo[1] = kMAlign;
                    }
                } else {
                    pg[0] = group_at(0);
                    if (pg[0] < 0) continue;
                }
            }
            return true;
        }
    };
    // the tile the hand-out state describes
    auto build_tile = [&](Tile& t) DG_INLINE {
        const int g = pass == 0 ? pg[0] : pg[1];
        const int m0 = st_m0, n0 = st_n0, valid_rows = st_vr;
        t.m0 = m0;
        t.grp = g;
        t.row_lo = pass == 0 ? plo[0] : plo[1];
        t.row_hi = min(pass == 0 ? phi[0] : phi[1], valid_rows);
        const uint8_t* a_tile = a_ptr + (LAYOUT == kMasked ? (long)g * p.a_gstride : 0) + (long)m0 * p.lda;
        const uint8_t* b_tile = b_ptr + (long)g * p.b_gstride + (long)n0 * p.ldb;
        const float* sa_tile = sa_ptr + (LAYOUT == kMasked ? (long)g * p.sa_gstride : 0) + m0;
        t.sb_grp = sb_ptr + (long)g * p.sb_gstride;
        t.d_tile = d_ptr + (LAYOUT == kMasked ? (long)g * p.d_gstride : 0) + (long)m0 * p.ldd;
        // Buffer descriptors over this tile's operands: the K offset of each stage
        // travels in a scalar register, so issuing a stage costs no vector ALU work.
        // Masked layout: rows at or past masked_m fall outside the descriptor, so their
        // copies return zeros without a memory access (their outputs are never stored).
        const int a_rows_read = LAYOUT == kMasked ? valid_rows : p.rows - m0;
        t.rs_a = make_rsrc(a_tile, (long)a_rows_read * p.lda);
        t.rs_b = make_rsrc(b_tile, (long)(NN - n0) * p.ldb);
        t.rs_sa = make_rsrc(sa_tile, ((long)KBT * p.ld_sa - m0) * 4);
        // Sub-tile column fn (MF columns, inside one 128-column scale block because MF
        // divides 128 and the column offsets are multiples of MF) reads its B scales
        // from row nb(fn) of sB; the byte offset of that row is wave-uniform.
        // With MF=16 a wave spans at most 128 columns, i.e. two scale rows (lo, hi):
        // two loads per K block and a per-column choice by a uniform bit mask.
        t.wcol0 = n0 + wn * WTN;
        t.hi_mask = 0;
        if constexpr (MF == 16) {
            const int nb_lo = min(t.wcol0 / kKBlock, NBLK - 1);
            t.sb_off[0] = nb_lo * KBT * 4;
            if constexpr (!ONE_SB) {
                t.sb_off[NSB - 1] = min(nb_lo + 1, NBLK - 1) * KBT * 4;
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    if ((t.wcol0 + fn * MF) / kKBlock > nb_lo) t.hi_mask |= 1u << fn;
            }
        } else {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                t.sb_off[fn] = min((t.wcol0 + fn * MF) / kKBlock, NBLK - 1) * KBT * 4;
        }
        t.active = wm * WTM < t.row_hi && wm * WTM + WTM > t.row_lo;
    };
    // no tile: its copies read nothing (every lane is out of range) and write zeros
    auto null_tile = [&](Tile& t) DG_INLINE {
        t.m0 = t.row_lo = t.row_hi = t.wcol0 = 0;
        t.grp = -1;
        t.hi_mask = 0;
#pragma unroll
        for (int i = 0; i < NSB; ++i) t.sb_off[i] = 0;
        t.active = false;
        t.rs_a = t.rs_b = t.rs_sa = make_rsrc(a_ptr, 0);
        t.sb_grp = sb_ptr;
        t.d_tile = d_ptr;
    };
    // move the hand-out state to the tile after the current one; false when none is left
    auto advance = [&]() DG_INLINE -> bool {
        if (pass + 1 < npass) {
            ++pass;
            return true;
        }
        ++step;
        pass = 0;
        return fetch_step();
    };

    Tile cur, nx;
    if (!fetch_step()) return;   // uniform: no work for this workgroup
    build_tile(cur);

    // DMA slot t of this wave (A slots first, then B slots) for K block kb of tile
    // tl.  A slot index past the last one repeats the last slot: the same bytes land
    // on the same LDS location twice, which keeps the issue free of branches.
    // B copies of the masked layout are non-temporal: the row block covers a group's
    // capacity, so each B tile is read by one workgroup, once (at most by the few row
    // blocks of one group, handed out side by side, when the capacity exceeds the row
    // block), and its lines then leave L2 first instead of the group's A rows, which
    // all of the group's tiles read.  Measured on 16 groups of 256 rows, N = 4096,
    // K = 7168: -12% with the seeded counts, -9% with full groups.  In the dense and
    // contiguous layouts every B and A tile is shared and the hint costs 5-30%.
    constexpr int B_CPOL = LAYOUT == kMasked ? kCpolNT : 0;
    // With K groups, step kb of the K loop holds K block kb*WK + wk of this wave's group
    // (its operand rows at sub-block wk of the stage); a block past the last one (K/128
    // odd) is copied from no memory, i.e. as zeros, and adds nothing.
    const __amdgpu_buffer_rsrc_t rs_none = make_rsrc(a_ptr, 0);
    auto kblock = [&](int kb) DG_INLINE { return WK == 1 ? kb : kb * WK + wk; };
    auto issue_slot = [&](const Tile& tl, uint8_t* smem, int kb, int t) DG_INLINE {
        const int kr = kblock(kb);
        const int koff = kr * kKBlock;
        uint8_t* const sub = smem + (WK == 1 ? 0 : wk * SUB);
        if (t < A_PER) {
            const int j = min(wg + t * NWG, A_SLOTS - 1);
            buffer_copy_lds16(WK == 1 || kr < KBT ? tl.rs_a : rs_none, (lds_void*)(sub + j * 1024), (int)a_off[t],
                              koff);
        } else {
            const int j = min(wg + (t - A_PER) * NWG, B_SLOTS - 1);
            buffer_copy_lds16<B_CPOL>(WK == 1 || kr < KBT ? tl.rs_b : rs_none,
                                      (lds_void*)(sub + BM * kKBlock + j * 1024), (int)b_off[t - A_PER], koff);
        }
    };
    // (past the last K block the offset lies outside the tile's sA descriptor: zeros)
    auto issue_sa = [&](const Tile& tl, uint8_t* smem, int kb) DG_INLINE {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tl.rs_sa,
                                                 (lds_void*)(smem + WK * SUB + wave * 256), 4,
                                                 (int)(sa_voff + (uint32_t)(kblock(kb) * p.ld_sa) * 4u), 0, 0, 0);
    };
    auto issue_stage = [&](const Tile& tl, uint8_t* smem, int kb) DG_INLINE {
#pragma unroll
        for (int t = 0; t < NSLOT; ++t) issue_slot(tl, smem, kb, t);
        issue_sa(tl, smem, kb);
    };

    // per-lane LDS byte offsets of the 16-byte chunks of this lane's fragment
    // (MF=16: chunks 2g, 2g+1 of the 128-K row; MF=32: chunks 4h+2g, 4h+2g+1 for
    // K half h), swizzled like the rows were written
    int coff[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            coff[h][e] = (((MF == 16 ? 2 * lgrp : 4 * h + 2 * lgrp) + e) ^ swz(lane & 15)) * 16;

    // Scales of one K block: a[fm] per lane (its row of sub-tile row fm), b[t]
    // wave-uniform (scalar loads of sB, which never pass through the texture unit)
    struct Scales { float a[FM]; float b[NSB]; };
    auto load_sb = [&](const Tile& tl, Scales& sc, int kb) DG_INLINE {
#pragma unroll
        for (int t = 0; t < NSB; ++t) sc.b[t] = tl.sb_grp[(tl.sb_off[t] >> 2) + (WK == 1 ? kb : min(kblock(kb), KBT - 1))];
    };
    auto read_sa = [&](Scales& sc, const uint8_t* smem) DG_INLINE {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            sc.a[fm] = *(const lds_f32*)((const lds_u8*)smem + sa_lds + fm * MF * 4);
    };
    // the B scale of sub-tile column fn as a scalar: MF=16 picks the wave's low or
    // high scale row with uniform integer operations
    auto pick_b = [&](const Scales& sc, int fn) DG_INLINE -> float {
        if constexpr (ONE_SB) {
            return sc.b[0];
        } else if constexpr (MF == 16) {
            const unsigned m = 0u - ((cur.hi_mask >> fn) & 1u);
            const unsigned lo = __builtin_bit_cast(unsigned, sc.b[0]);
            const unsigned hi = __builtin_bit_cast(unsigned, sc.b[NSB - 1]);
            return __builtin_bit_cast(float, lo ^ ((lo ^ hi) & m));
        } else {
            return sc.b[fn];
        }
    };

    // ---- K loop: one continuous stream of steps over (K block, column fn, row fm).
    // Step j of a block issues the MFMA(s) of sub-tile (fm, fn) = (j % FM, j / FM)
    // and promotes the partial of the step kLag earlier, which may belong to the
    // previous K block (its scales are still held), so the matrix core never
    // waits for a promotion and a block boundary costs no pipeline drain.
    // LDS stages: block kb lives in stage kb % NST.  In each block the single
    // workgroup barrier sits at step JB, shortly after the last read of this block's
    // stage (16x16 sub-tiles: two steps after it, or, with the B fragment ring, at the
    // first read of the next block's stage; the first MFMA of the last column for 32x32).
    // By then every wave has finished reading this block's stage, except for the
    // fragments already in registers, and has waited for its own copies of the
    // next block, so after the barrier
    //   * the next block's fragments are read while the last column's MFMAs run
    //     (each A fragment as soon as its last MFMA of this block is issued), and
    //   * the stage read in this block is free: the copies of block kb + NST go
    //     there, issued every other step and running on into the next block.
    // When K/128 is a multiple of NST, the blocks past the last one are the next
    // tile's first blocks: their copies, A scales and fragments arrive while this
    // tile finishes, so a tile boundary costs no pipeline refill either.
    constexpr int NJ = FN * FM;
    // ring of in-flight partials: its position is a compile-time function of the
    // step because the block loop is unrolled by NST
    constexpr int R = MF == 32 ? 2
                    : ((NST * NJ) % 4 == 0 ? 4 : ((NST * NJ) % 3 == 0 ? 3 : 2));
    static_assert((NST * NJ) % R == 0, "partial ring must tile the unrolled loop");
    constexpr int kLag = R - 1;
    // B fragments are read ahead of their column: one column ahead when a column has
    // three or more MFMAs (FM >= 3) to cover the LDS read; with fewer, PDC columns
    // ahead into a ring of PDC + 1 registers, so that every read still has about three
    // MFMAs to land.  Ring slot of column c of the block in stage U: (U*FN + c) % RB.
    // (Shortened where a longer ring would not tile the loop unrolled over NST blocks,
    // or would put the barrier before the promotions that still need the previous
    // block's scales.)
    constexpr int PDC = [] {
        if (!(MF == 16 && FM <= 2)) return 1;
        int d = (3 + FM - 1) / FM < FN - 1 ? (3 + FM - 1) / FM : FN - 1;
        while (d > 1 && ((NST * FN) % (d + 1) != 0 || (FN - d) * FM < kLag)) --d;
        return d;
    }();
    constexpr bool BRING = PDC > 1;
    constexpr int RB = PDC + 1;
    static_assert(!BRING || (NST * FN) % RB == 0, "B fragment ring must tile the unrolled loop");
    // (the last read of this block's stage is the B fragment of the last column, at
    // the first step of column FN-1-PDC; the barrier sits at or before the step whose
    // read-ahead first reaches the next block's stage (column FN-PDC); for FM >= 3 an
    // earlier barrier spreads the next block's first reads over more steps)
    constexpr int EARLY = MF == 16 && FM > 2 ? FM - 2 : 0;
    constexpr int JB = BRING ? (FN - PDC) * FM : (FN - 1) * FM - EARLY;
    static_assert(FN >= 2, "the barrier sits in the last of at least two columns");
    constexpr int NVM = NSLOT + 1;             // vector memory instructions per block
    // Copies of block kb + NST (NSLOT operand slots, then the A-scale copy) go to
    // stage kb % NST as soon as block kb's barrier has freed it: copy t at step
    // JB + 1 + t*CPN/CPD of block kb (two steps apart when a block is long enough),
    // running on into the first steps of block kb+1, never past its barrier
    // (where, for NST=2, they must have landed).  The masked layout streams B
    // with little MFMA work per byte, so there the copies go out one step apart:
    // the last one leaves earlier and has longer to land before the barrier.
    constexpr int NDMA = NSLOT + 1;
    constexpr int CPN = LAYOUT == kMasked ? 1 : (2 * NDMA + 4 <= NJ ? 2 : (NDMA + 4 <= NJ ? 1 : NJ));
    constexpr int CPD = CPN == NJ ? NDMA : 1;
    static_assert((NDMA - 1) * CPN / CPD + 1 <= NJ, "copies must be issued before the next barrier");
    constexpr int NFIRST = [] {   // copies issued in the freeing block
        int c = 0;
        for (int t = 0; t < NDMA; ++t) c += JB + 1 + t * CPN / CPD < NJ;
        return c;
    }();
    static_assert(kLag <= JB, "the previous block's scales are dead by the barrier");
    // copy t of block kb of tile tl into stage smem (blocks past the last one of a
    // tile that is not followed by pipelined work re-read block KB-1)
    auto issue_copy = [&](const Tile& tl, int t, uint8_t* smem, int kb) DG_INLINE {
        if (t < NSLOT) issue_slot(tl, smem, kb, t);
        else issue_sa(tl, smem, kb);
    };

    Scales sc[NST];
    // stage i's buffer; every index is a compile-time constant (no array of stage
    // pointers exists, so nothing can index one at run time)
    auto stage = [&](auto idx) -> uint8_t* {
        constexpr int i = decltype(idx)::value;
        static_assert(i >= 0 && i < NST, "stage index");
        if constexpr (i == 0) return smem0;
        else if constexpr (i == 1) return smem1;
        else if constexpr (i == 2) return smem2;
        else if constexpr (i == 3) return smem3;
        else if constexpr (i == 4) return smem4;
        else if constexpr (i == 5) return smem5;
        else if constexpr (i == 6) return smem6;
        else return smem7;
    };
    using std::integral_constant;
    constexpr int NH = MF == 32 ? 2 : 1;
    v8i af[FM][NH], bf[NH], bnext;
    v8i bq[RB];                                // B fragment ring (BRING)
    vacc part[R];
    vacc acc[FM][FN];
    const int arow0 = wk * ROWS + wm * WTM, bcol0 = wk * ROWS + BM + wn * WTN;   // (ROWS is a multiple of 16)

    // This lane's byte offsets in a stage from the first row of the wave's A or B
    // rows, made opaque to the compiler so that every fragment read is stage +
    // offset + an immediate row offset (no per-read address arithmetic, and no
    // separately hoisted address register per fragment and stage).  Only the
    // offset is hidden: the stage array stays visible, so the compiler knows
    // which stage a read touches and that it is not one the copies fill.
    auto lane_base = [&](const uint8_t* smem, int row_base, lds_u8* (&lb)[2][2]) DG_INLINE {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                int off = (row_base + lsub) * kKBlock + coff[h][e];
                asm volatile("" : "+v"(off));
                lb[h][e] = (lds_u8*)smem + off;
            }
    };
    // fragment of sub-tile rows [row0, row0+MF) past the lane base's first row, for
    // K half h (MF=16: whole block)
    auto frag = [&](lds_u8* const (&lb)[2][2], int row0, int h) DG_INLINE -> v8i {
        const v4i lo = *(const lds_v4i*)(lb[h][0] + row0 * kKBlock);
        const v4i hi = *(const lds_v4i*)(lb[h][1] + row0 * kKBlock);
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    // the first block's fragments and scales of a tile, from stage 0 (read in the
    // order the loop issues a next block's reads: B fragment, A scales, A fragments)
    auto first_fragments = [&]() DG_INLINE {
        lds_u8* la[2][2];
        lds_u8* lb[2][2];
        lane_base(smem0, arow0, la);
        lane_base(smem0, bcol0, lb);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if constexpr (BRING) {
#pragma unroll
                for (int c = 0; c < PDC; ++c) bq[c] = frag(lb, c * MF, 0);
            } else {
                bf[h] = frag(lb, 0, h);
            }
            if (h == 0) read_sa(sc[0], smem0);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) af[fm][h] = frag(la, fm * MF, h);
        }
    };
    // tile start: the "previous block" of block 0 has zero partials and zero scales
    auto reset_tile = [&]() DG_INLINE {
#pragma unroll
        for (int r = 0; r < R; ++r) part[r] = vacc{};
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) sc[NST - 1].a[fm] = 0.f;
#pragma unroll
        for (int t = 0; t < NSB; ++t) sc[NST - 1].b[t] = 0.f;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = vacc{};
    };

    // ---- prologue of the first tile: copies of blocks 0 .. NST-2 and the early
    // part of block NST-1's (clamped), then the first block's fragments and scales ----
    auto prologue = [&](const Tile& tl) DG_INLINE {
        static_for<0, NST - 1>([&](auto ss) DG_INLINE {
            constexpr int s = decltype(ss)::value;
            issue_stage(tl, stage(ss), s < KB ? s : KB - 1);
        });
#pragma unroll
        for (int t = 0; t < NFIRST; ++t)
            issue_copy(tl, t, stage(integral_constant<int, NST - 1>{}), NST - 1 < KB ? NST - 1 : KB - 1);
        // (the scalar loads complete before the loop, so the loop starts with only LDS
        // reads in flight)
        if (tl.active) load_sb(tl, sc[0], 0);
        wait_lds_all();
        wait_vmem_le<(NST - 2) * NVM + NFIRST>();
        stage_barrier();
        if (tl.active) first_fragments();
    };
    prologue(cur);

    // One K block (stage U of the unrolled loop, block index kbu).  TAIL: one of the
    // last NST blocks of a tile whose K/128 is a multiple of NST; its copies past
    // the last block go to the next tile `nx` (blocks kb - KB; a null tile reads
    // nothing).  Otherwise copies past the last block re-read block KB-1.
    auto block = [&](auto stage_tag, auto tail_tag, int kbu) DG_INLINE {
        constexpr int U = decltype(stage_tag)::value;
        constexpr bool TAIL = decltype(tail_tag)::value;
        uint8_t* const curs = stage(integral_constant<int, U>{});
        const uint8_t* nxt = stage(integral_constant<int, (U + 1) % NST>{});
        uint8_t* dst = stage(integral_constant<int, (U + NST - 1) % NST>{});
        const Scales& scs = sc[U];
        const Scales& scp = sc[(U + NST - 1) % NST];   // previous block's
        Scales& scn = sc[(U + 1) % NST];               // next block's (for NST=2: scp's slot)
        lds_u8* lc[2][2];    // B rows of this block's stage
        lds_u8* ln[2][2];    // B rows of the next block's stage
        lds_u8* lna[2][2];   // A rows of the next block's stage
        lane_base(curs, bcol0, lc);
        lane_base(nxt, bcol0, ln);
        lane_base(nxt, arow0, lna);
        auto scale = [&](bool prev, int fm, int fn) DG_INLINE {
            const Scales& sc = prev ? scp : scs;
            return sc.a[fm] * pick_b(sc, fn);
        };
        auto promote = [&](int q, int i0, int i1) DG_INLINE {
            // q: step index relative to this block, possibly negative (previous block)
            const int slot = ((U * NJ + q) % R + R) % R;
            const int qq = q < 0 ? q + NJ : q;
            const float s = scale(q < 0, qq % FM, qq / FM);
            const vacc& pq = part[slot];
#pragma unroll
            for (int i = i0; i < i1; ++i)
                acc[qq % FM][qq / FM][i] = __builtin_fmaf(pq[i], s, acc[qq % FM][qq / FM][i]);
        };
        // copy t of block kb (>= kbu): of this tile, of the next one in the tail, or a
        // re-read of block KB-1
        auto copy = [&](int t, uint8_t* smem, int kb, bool past) DG_INLINE {
            if constexpr (TAIL) {
                if (past) issue_copy(nx, t, smem, kb - KB);
                else issue_copy(cur, t, smem, kb);
            } else {
                issue_copy(cur, t, smem, kb < KB ? kb : KB - 1);
            }
        };
        auto issue_loads = [&](int j) DG_INLINE {
#pragma unroll
            for (int t = 0; t < NDMA; ++t) {
                const int g = JB + 1 + t * CPN / CPD;
                // in the tail every block's first-part copies are past the end, and its
                // wrapped copies are past the end except in the tail's first block
                if (g < NJ && j == g) copy(t, curs, kbu + NST, true);
                if (g >= NJ && j == g - NJ) copy(t, dst, kbu + NST - 1, U > 0);
            }
        };
        auto barrier = [&]() DG_INLINE {
            // The next block's B scales (scalar loads) are issued here, where the
            // wave waits for all its LDS reads anyway: scalar loads complete out of
            // order and share that counter, so while one is in flight every wait
            // for an LDS read would have to be a wait for all of them.  The slot's
            // previous contents were last used by promotions early in this block.
            // The tail's last block loads the next tile's block 0 (if any).
            if constexpr (TAIL && U == NST - 1) {
                load_sb(nx, scn, 0);
            } else {
                load_sb(cur, scn, kbu + 1 < KB ? kbu + 1 : KB - 1);
            }
            wait_lds_all();
            wait_vmem_le<(NST - 2) * NVM>();
            stage_barrier();
        };
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int fn = j / FM, fm = j % FM;
            const int slot = (U * NJ + j) % R;
            if constexpr (MF == 16 && BRING) {
                part[slot] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bq[(U * FN + fn) % RB], af[fm][0], vacc{},
                                                                              FMT_SRC0, FMT_SRC1, 0, 0, 0, 0);
                promote(j - kLag, 0, NACC);
                issue_loads(j);
                if (j == JB) barrier();
                // column fn + PDC (of the next block's stage past the last column), into
                // the slot of column fn - 1, whose MFMAs are all issued
                if (fm == 0) {
                    const int c = fn + PDC;
                    bq[(U * FN + c) % RB] = c < FN ? frag(lc, c * MF, 0) : frag(ln, (c - FN) * MF, 0);
                }
                if (j == JB) read_sa(scn, nxt);
                if (fn == FN - 1) af[fm][0] = frag(lna, fm * MF, 0);
            } else if constexpr (MF == 16) {
                part[slot] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[0], af[fm][0], vacc{}, FMT_SRC0, FMT_SRC1,
                                                                              0, 0, 0, 0);
                promote(j - kLag, 0, NACC);
                issue_loads(j);
                if (j == JB) barrier();
                if (fm == 0) bnext = fn + 1 < FN ? frag(lc, (fn + 1) * MF, 0) : frag(ln, 0, 0);
                if (j == JB) read_sa(scn, nxt);
                if (fn == FN - 1) af[fm][0] = frag(lna, fm * MF, 0);
                if (fm == FM - 1) bf[0] = bnext;
            } else {
                part[slot] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[0], af[fm][0], vacc{}, FMT_SRC0, FMT_SRC1,
                                                                             0, 0, 0, 0);
                promote(j - kLag, 0, NACC / 2);
                issue_loads(j);
                if (j == JB) barrier();
                // each K half's fragments are reloaded as soon as the MFMA that
                // reads them for the last time in this block has been issued
                if (fm == FM - 1) bf[0] = fn + 1 < FN ? frag(lc, (fn + 1) * MF, 0) : frag(ln, 0, 0);
                if (j == JB) read_sa(scn, nxt);
                if (fn == FN - 1) af[fm][0] = frag(lna, fm * MF, 0);
                __builtin_amdgcn_sched_barrier(0);
                part[slot] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[1], af[fm][1], part[slot], FMT_SRC0,
                                                                             FMT_SRC1, 0, 0, 0, 0);
                promote(j - kLag, NACC / 2, NACC);
                if (fm == FM - 1) bf[1] = fn + 1 < FN ? frag(lc, (fn + 1) * MF, 1) : frag(ln, 0, 1);
                if (fn == FN - 1) af[fm][1] = frag(lna, fm * MF, 1);
            }
            // keep this order: the scheduler would otherwise pull each promotion up
            // against its own MFMA and stall on the result
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the partials of the last block's final kLag steps, promoted after the loop
    auto drain = [&](auto stage_tag) DG_INLINE {
        constexpr int U = decltype(stage_tag)::value;
        const Scales& sl = sc[U];
#pragma unroll
        for (int q = NJ - kLag; q < NJ; ++q) {
            const int fm = q % FM, fn = q / FM;
            const float s = sl.a[fm] * pick_b(sl, fn);
            const vacc& pq = part[(U * NJ + q) % R];
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[fm][fn][i] = __builtin_fmaf(pq[i], s, acc[fm][fn][i]);
        }
    };
    // PIPE (chosen by the host when K/128 is a multiple of NST): a tile's blocks past
    // its last one are the next tile's first blocks
    reset_tile();

    for (;;) {
        // the next tile's position is known from here on; its descriptors are built
        // only where its copies start, which keeps them out of the hot loop's registers
        const bool has_nx = advance();
        const bool piped = PIPE && has_nx;
        auto make_nx = [&]() DG_INLINE {
            if (has_nx) build_tile(nx);
            else null_tile(nx);
        };
        if (cur.active) {
            // whole groups of NST blocks (the last group is the tail when K/128 is a
            // multiple of NST), then the remaining KB % NST blocks: the hot loop has a
            // single exit, which keeps the register allocator from splitting the
            // accumulators' live ranges around mid-body exits
            const int KF = KB - KB % NST;
            if constexpr (PIPE) {
                const int KM = KF - NST;
                for (int kb = 0; kb < KM; kb += NST)
                    static_for<0, NST>([&](auto u) DG_INLINE { block(u, std::false_type{}, kb + decltype(u)::value); });
                make_nx();
                static_for<0, NST>([&](auto u) DG_INLINE { block(u, std::true_type{}, KM + decltype(u)::value); });
            } else {
                for (int kb = 0; kb < KF; kb += NST)
                    static_for<0, NST>([&](auto u) DG_INLINE { block(u, std::false_type{}, kb + decltype(u)::value); });
                static_for<0, NST - 1>([&](auto u) DG_INLINE {
                    if (KF + decltype(u)::value < KB) block(u, std::false_type{}, KF + decltype(u)::value);
                });
            }
            const int ul = (KB - 1) % NST;
            static_for<0, NST>([&](auto u) DG_INLINE {
                if (ul == decltype(u)::value) drain(u);
            });
        } else {
            // a wave with no valid rows (masked / short tiles) still copies its share
            // of every stage (operands and A scales) and meets every barrier; copies
            // past the last block feed the next tile when it is pipelined
            if constexpr (PIPE) make_nx();
            for (int kb = 0; kb < KB; kb += NST) {
                static_for<0, NST>([&](auto uu) DG_INLINE {
                    constexpr int u = decltype(uu)::value;
                    if (kb + u < KB) {
                        uint8_t* const st = stage(integral_constant<int, (u + NST - 1) % NST>{});
                        const int b = kb + u + NST - 1;
                        if (b < KB) issue_stage(cur, st, b);
                        else if (piped) issue_stage(nx, st, b - KB);
                        else issue_stage(cur, st, KB - 1);
                        wait_vmem_le<(NST - 2) * NVM>();
                        stage_barrier();
                    }
                });
            }
            // ... and, like the tail of an active wave, the early copies of the next
            // tile's block NST-1
            if (piped) {
#pragma unroll
                for (int t = 0; t < NFIRST; ++t) issue_copy(nx, t, stage(integral_constant<int, NST - 1>{}), NST - 1);
            }
        }

        // ---- epilogue: BF16 RNE, skip padding / masked / tail rows.  A lane owns row
        // lsub of each sub-tile and runs of four adjacent columns (MF=16: columns
        // 4g..4g+3 of lane group g; MF=32: columns 8q+4g..8q+4g+3, q = 0..3).  MF=16:
        // for each pair of sub-tile columns, two lane-group swaps (V_PERMLANE16_SWAP)
        // give every lane eight adjacent columns of one sub-tile, so a store
        // instruction writes 64 contiguous bytes per row in 16-byte pieces. ----
        if constexpr (WK > 1) {
            // K groups: group 1 leaves its sums in LDS (stage 0, free once every copy has
            // landed and every wave has passed the barrier), group 0 adds them to its own
            constexpr int NV = FM * FN * NACC;       // accumulator floats per lane
            static_assert(ROWS % 16 == 0, "sub-blocks keep the fragment swizzle");
            static_assert(NWG * NV * 64 * 4 <= STAGE, "one K group's sums fit a stage");
            typedef __attribute__((address_space(3))) float lds_f32w;
            lds_f32w* const red = (lds_f32w*)(lds_u8*)smem0 + wg * NV * 64 + lane;
            wait_vmem_le<0>();
            __syncthreads();
            if (cur.active && wk == 1) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int i = 0; i < NACC; ++i) red[((fm * FN + fn) * NACC + i) * 64] = acc[fm][fn][i];
            }
            __syncthreads();
            if (cur.active && wk == 0) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int i = 0; i < NACC; ++i) acc[fm][fn][i] += red[((fm * FN + fn) * NACC + i) * 64];
            }
        }
        if (cur.active && wk == 0) {
            auto pack2 = [](float x, float y) DG_INLINE -> uint32_t {
                typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
                const v2bf t = {(__bf16)x, (__bf16)y};
                return __builtin_bit_cast(uint32_t, t);
            };
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int lr = wm * WTM + fm * MF + lsub;     // row inside the tile
                bool row_ok = lr >= cur.row_lo && lr < cur.row_hi;
                if constexpr (LAYOUT == kContiguous) {
                    // only rows of this pass's group: padding (-1) and entries that
                    // break the one-group-per-segment-block rule are not written
                    if (row_ok) row_ok = p.m_indices[cur.m0 + lr] == cur.grp;
                }
                uint16_t* drow = cur.d_tile + (long)(row_ok ? lr : 0) * p.ldd;
                if constexpr (MF == 16) {
#pragma unroll
                    for (int fn = 0; fn + 1 < FN; fn += 2) {
                        const vacc& x = acc[fm][fn];
                        const vacc& y = acc[fm][fn + 1];
                        // every lane takes part in the swaps; only the stores are predicated
                        const auto s0 = __builtin_amdgcn_permlane16_swap(pack2(x[0], x[1]), pack2(y[0], y[1]), false,
                                                                         false);
                        const auto s1 = __builtin_amdgcn_permlane16_swap(pack2(x[2], x[3]), pack2(y[2], y[3]), false,
                                                                         false);
                        // lane group g now holds sub-tile fn + (g & 1), columns 8*(g >> 1) .. +7
                        const int col = cur.wcol0 + (fn + (lgrp & 1)) * MF + (lgrp >> 1) * 8;
                        if (row_ok && (WHOLE_N || col < NN)) *(uint4*)(drow + col) = uint4{s0[0], s1[0], s0[1], s1[1]};
                    }
                    if constexpr (FN % 2 == 1) {
                        const vacc& x = acc[fm][FN - 1];
                        const int col = cur.wcol0 + (FN - 1) * MF + lgrp * 4;
                        if (row_ok && (WHOLE_N || col < NN)) *(uint2*)(drow + col) = uint2{pack2(x[0], x[1]), pack2(x[2], x[3])};
                    }
                } else {
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                        for (int q = 0; q < NACC / 4; ++q) {
                            const int col = cur.wcol0 + fn * MF + q * 8 + lgrp * 4;
                            if (row_ok && (WHOLE_N || col < NN))
                                *(uint2*)(drow + col) = uint2{pack2(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1]),
                                                              pack2(acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3])};
                        }
                    }
                }
            }
        }

        if constexpr (PIPE) {
            if (!has_nx) break;
            // The next tile's first blocks are already in LDS (certified by this tile's
            // last barrier), and an active wave has its first fragments and scales in
            // registers; a wave that was idle reads them now.
            const bool was_active = cur.active;
            cur = nx;
            reset_tile();
            if (cur.active && !was_active) {
                load_sb(cur, sc[0], 0);
                first_fragments();
            }
        } else {
            // the copies issued past the last K block must land before the next tile
            // (or another workgroup) reuses these buffers; then every wave is done
            wait_vmem_le<0>();
            __syncthreads();
            if (!has_nx) break;
            build_tile(cur);
            reset_tile();
            prologue(cur);
        }
    }
    // the last tile's copies past its end (of nothing) land before the exit
    if constexpr (PIPE) wait_vmem_le<0>();
}

template <int BM, int BN, int WM, int WN, int LAYOUT, int MF, int NST, bool PIPE, int FMT, int WK, int NC = 0,
          int KC = 0>
static hipError_t launch_one(const GemmParams& p, int grid, hipStream_t s) {
    hipLaunchKernelGGL((dg_gemm_kernel<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE, FMT, NC, KC, WK>), dim3(grid),
                       dim3(WM * WN * WK * 64), 0, s, p, p.a, p.sa, p.b, p.sb, p.d);
    return hipGetLastError();
}

// The instance for operand formats FMT: the one compiled for the call's N and K when
// the configuration has shape instances (SPEC) and kSpecShapes lists them for its
// layout; pipelined (the next tile's first NST blocks run as the tail of the current
// one) when K/128 splits into whole groups of NST and the configuration fits that
// variant's registers (PIPE_OK); else the generic per-tile loop.
template <int BM, int BN, int WM, int WN, int LAYOUT, int MF, int NST, bool PIPE_OK, bool SPEC, int FMT, int WK>
static hipError_t launch_fmt(const GemmParams& p, int grid, hipStream_t s) {
    if constexpr (SPEC) {
        bool done = false;
        hipError_t e = hipSuccess;
        static_for<0, kNumSpecShapes>([&](auto i) {
            constexpr SpecShape sh = kSpecShapes[decltype(i)::value];
            if constexpr (sh.grouped == (LAYOUT != kDense)) {
                constexpr bool PIPE = PIPE_OK && sh.kblocks % NST == 0;
                if (!done && p.n == sh.n && p.kblocks == sh.kblocks) {
                    e = launch_one<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE, FMT, WK, sh.n, sh.kblocks>(p, grid, s);
                    done = true;
                }
            }
        });
        if (done) return e;
    }
    if constexpr (PIPE_OK) {
        if (p.kblocks % NST == 0) return launch_one<BM, BN, WM, WN, LAYOUT, MF, NST, true, FMT, WK>(p, grid, s);
    }
    return launch_one<BM, BN, WM, WN, LAYOUT, MF, NST, false, FMT, WK>(p, grid, s);
}

// Configurations with ALL_FMT have instances for the four operand-format pairs (E5M2 on
// either side); the planner gives the others E4M3 operands only.
template <int BM, int BN, int WM, int WN, int LAYOUT, int MF, int NST, bool PIPE_OK, bool ALL_FMT, bool SPEC, int WK>
static hipError_t launch_cfg(const GemmParams& p, int grid, hipStream_t s) {
    if constexpr (ALL_FMT) {
        switch (p.fmt) {
            case 1: return launch_fmt<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, SPEC, 1, WK>(p, grid, s);
            case 2: return launch_fmt<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, SPEC, 2, WK>(p, grid, s);
            case 3: return launch_fmt<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, SPEC, 3, WK>(p, grid, s);
            default: break;
        }
    }
    if (p.fmt != 0) return hipErrorInvalidValue;
    return launch_fmt<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, SPEC, 0, WK>(p, grid, s);
}

template <int BM, int BN, int WM, int WN, int LAYOUT, int MF, int NST, bool PIPE_OK, int WK>
static hipError_t occupancy_cfg(int* blocks) {
    typedef void (*KernelFn)(const GemmParams, const uint8_t*, const float*, const uint8_t*, const float*, uint16_t*);
    const KernelFn k0 = dg_gemm_kernel<BM, BN, WM, WN, LAYOUT, MF, NST, false, 0, 0, 0, WK>;
    const KernelFn k1 = dg_gemm_kernel<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, 0, 0, 0, WK>;
    int b0 = 0, b1 = 0;
    constexpr int threads = WM * WN * WK * 64;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b0, reinterpret_cast<const void*>(k0), threads, 0);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b1, reinterpret_cast<const void*>(k1), threads, 0);
    *blocks = b0 < b1 ? b0 : b1;
    return e;
}

#define DG_CFG(ID, LAYOUT, BM, BN, WM, WN, WK, MF, NST, EFF, PIPE_OK, ALL_FMT, SPEC)                           \
    {ID, LAYOUT, BM, BN, WM, WN, WK, EFF, ALL_FMT, SPEC,                                                        \
     &launch_cfg<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, ALL_FMT, SPEC, WK>,                                  \
     &occupancy_cfg<BM, BN, WM, WN, LAYOUT, MF, NST, PIPE_OK, WK>},

static const KernelConfig kConfigs[] = {DG_CONFIG_TABLE(DG_CFG)};

const KernelConfig* kernel_configs(int* count) {
    *count = (int)(sizeof(kConfigs) / sizeof(kConfigs[0]));
    return kConfigs;
}

}  // namespace dg
