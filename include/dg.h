/*
 * dg.h -- C ABI of the MI355X (gfx950) fine-grained-scaled FP8 E4M3 "NT" GEMM
 * library (libdg.so).
 *
 * The operation (all three layouts reduce to it), from "DeepGEMM: clean and
 * efficient FP8 GEMM kernels with fine-grained scaling" (nipponese.news
 * translation of the project README), intro and usage paragraphs:
 *
 *     D[m, n] = bf16( sum_kb  sA[m, kb] * sB[n / 128, kb] * sum_{k in kb} A[m, k] * B[n, k] )
 *
 *   A  : E4M3 (OCP E4M3FN bytes), [M, K] row-major, K contiguous ("non-transposed LHS")
 *   B  : E4M3, [N, K] row-major, K contiguous ("transposed RHS"); only NT is supported
 *   sA : fp32, one scale per (row, 128-wide K block), stored MN-major (the README's
 *        "LHS scaling factors must be transposed"): sa[kb * ld_sa + m]
 *   sB : fp32, one scale per (128-row N block, 128-wide K block): sb[nb * (K/128) + kb]
 *   D  : BF16 bits, [M, N] row-major, round-to-nearest-even from the fp32 accumulator
 *
 * Each K block's partial product is multiplied by sA*sB and added into an fp32
 * accumulator, K blocks in ascending order (the README's two-level "promotion";
 * the per-1x128 / per-128x128 granularity is DeepSeek-V3's fine-grained scheme).
 * One exception, dense calls only: where the tiles leave CUs idle and K/128 >= 32
 * (few rows, long K), the even and the odd K blocks are summed in two such chains
 * whose fp32 sums are added at the end; the result then agrees with the one-chain
 * result to fp32 rounding but need not be bit-identical to it.
 *
 * Conventions for every entry point:
 *  - Pointers named a, sa, b, sb, d, m_indices, masked_m are DEVICE pointers owned by
 *    the caller.  The library never allocates, frees, synchronises or reads device
 *    memory on the host, so every call is asynchronous on `stream` and may be
 *    captured into a hipGraph.  `stream` is a hipStream_t (NULL = default stream).
 *  - The return value reports host-side validation and launch errors only
 *    (DG_OK on success).  Nothing is launched when validation fails.
 *  - Requirements checked on the host: non-null pointers for non-empty problems;
 *    K > 0 and K % 128 == 0 (else DG_ERR_UNSUPPORTED); N % 16 == 0 (else
 *    DG_ERR_UNSUPPORTED); a, b, d, sa, sb 16-byte aligned; lda, ldb multiples of 16
 *    and >= K; ldd a multiple of 8 and >= N; ld_sa a multiple of 4 and >= the row
 *    count (else DG_ERR_MISALIGNED / DG_ERR_INVALID_ARG).
 *  - Size limits (else DG_ERR_UNSUPPORTED): 256 * lda + K and 256 * ldb + K below
 *    2^32 bytes, (K / 128) * ld_sa * 4 + 4096 below 2^32 bytes (for the grouped
 *    layouts lda = ldb = K), M * ldd * 4 below 2^63, and fewer than 2^30 output tiles;
 *    the kernels address each tile's operands through 32-bit offsets from the tile's
 *    first row.
 *  - M == 0 (or all masked_m == 0) is a valid no-op.
 *  - Calls on distinct streams may run concurrently; the only library state is the
 *    CU cap (dg_set_num_cus) and a per-device property cache.
 *  - Tuning and introspection hooks that are not part of this contract (pinning a
 *    tile configuration, listing the compiled ones, describing a launch) are declared
 *    in dg_tuning.h.
 */
#ifndef DG_H
#define DG_H

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = -1,   /* null pointer, negative size, leading dimension too small */
    DG_ERR_UNSUPPORTED = -2,   /* shape outside what the kernels handle (K % 128, N % 16, size limits) */
    DG_ERR_MISALIGNED = -3,    /* pointer or leading dimension alignment */
    DG_ERR_HIP = -4            /* a HIP runtime call or the kernel launch failed */
};

/* FP8 operand formats (dg_gemm_fp8_nt_fmt). */
enum {
    DG_FMT_E4M3 = 0,           /* OCP E4M3FN: max 448, no infinities */
    DG_FMT_E5M2 = 1            /* OCP E5M2: max 57344, infinities */
};

/* Human-readable name of a status code.  Never NULL; the string is static. */
const char* dg_status_string(int status);

/* Row alignment that every expert segment of the contiguous layout must be padded
 * to (the README's contiguous-layout paragraph: segments aligned to the GEMM
 * M-block size).  Always 128. */
int dg_get_m_alignment(void);

/* Cap on the number of compute units the GEMM kernels spread over (the README's
 * utility functions set_num_sms / get_num_sms).  n == 0 removes the cap; n < 0 is
 * DG_ERR_INVALID_ARG.  Returns DG_OK.  Process-wide. */
int dg_set_num_cus(int n);

/* The CU count the kernels will use on the current device: the cap if one is set
 * and smaller, else the device's CU count.  Returns a negative status if no HIP
 * device is usable and no cap is set. */
int dg_get_num_cus(void);

/* Dense NT GEMM (the README's basic non-grouped gemm_fp8_fp8_bf16_nt).
 *   a  [m][lda]          E4M3, K-major           b  [n][ldb]        E4M3, K-major
 *   sa [k/128][ld_sa]    fp32, MN-major          sb [ceil(n/128)][k/128] fp32
 *   d  [m][ldd]          BF16 bits (uint16)
 * All rows 0..m-1 and columns 0..n-1 of d are written; nothing else is. */
int dg_gemm_fp8_nt(const void* a, long lda,
                   const float* sa, long ld_sa,
                   const void* b, long ldb,
                   const float* sb,
                   void* d, long ldd,
                   int m, int n, int k, void* stream);

/* The dense NT GEMM with each operand's FP8 format chosen: DG_FMT_E4M3 or
 * DG_FMT_E5M2 for a and for b independently (the hnwysp.cn DeepGEMM blog,
 * section 2.3, lists E4M3 and E5M2 as the FP8 operand formats).  Scales, layouts,
 * promotion and output are exactly those of dg_gemm_fp8_nt, which is this call
 * with two E4M3 operands.  An unknown format is DG_ERR_INVALID_ARG.  E5M2
 * operands run on a subset of the tile configurations. */
int dg_gemm_fp8_nt_fmt(const void* a, long lda, const float* sa, long ld_sa,
                       const void* b, long ldb, const float* sb,
                       void* d, long ldd, int m, int n, int k,
                       int a_fmt, int b_fmt, void* stream);

/* M-grouped GEMM, contiguous layout (the README's contiguous-layout paragraph:
 * experts share N and K; their token segments are concatenated along M and each
 * segment is padded to dg_get_m_alignment() rows).
 *   a  [m_total][k]  E4M3          sa [k/128][ld_sa] fp32 MN-major (ld_sa >= m_total)
 *   b  [G][n][k]     E4M3          sb [G][ceil(n/128)][k/128] fp32
 *   d  [m_total][n]  BF16 bits
 *   m_indices [m_total] int32: the group of each row, or -1 for a padding row.
 * Device-side precondition (not checked by this call, which never reads m_indices on
 * the host; dg_check_contiguous_layout checks a host copy): within each aligned
 * 128-row block every non-negative entry is the group of the block's first row, and
 * the first row is padding only if the whole block is.  Only rows whose entry equals
 * their block's group are written; rows with -1 are not.
 * m_total must be a multiple of 128 (DG_ERR_INVALID_ARG otherwise). */
int dg_m_grouped_gemm_fp8_contiguous(const void* a, const float* sa, long ld_sa,
                                     const void* b, const float* sb,
                                     void* d, const int* m_indices,
                                     int m_total, int n, int k, int num_groups,
                                     void* stream);

/* M-grouped GEMM, masked layout (the README's masked-layout paragraph: for decode
 * under graph capture, where the host does not know how many rows each expert
 * received; only the valid rows are computed).
 *   a  [G][max_m][k]  E4M3         sa [G][k/128][ld_sa] fp32 MN-major (ld_sa >= max_m)
 *   b  [G][n][k]      E4M3         sb [G][ceil(n/128)][k/128] fp32
 *   d  [G][max_m][n]  BF16 bits
 *   masked_m [G] int32 (device): valid rows of each group, clamped to [0, max_m]
 *   on the device.  Rows >= masked_m[g] of d are never written (bit-exact). */
int dg_m_grouped_gemm_fp8_masked(const void* a, const float* sa, long ld_sa,
                                 const void* b, const float* sb,
                                 void* d, const int* masked_m,
                                 int num_groups, int max_m, int n, int k,
                                 void* stream);

/* The two grouped GEMMs with each operand's FP8 format chosen (DG_FMT_E4M3 or
 * DG_FMT_E5M2 for a and for b, as in dg_gemm_fp8_nt_fmt, after the same blog
 * section).  Everything else is exactly the call without _fmt, which is this
 * call with two E4M3 operands.  An unknown format is DG_ERR_INVALID_ARG; E5M2
 * operands run on a subset of the tile configurations. */
int dg_m_grouped_gemm_fp8_contiguous_fmt(const void* a, const float* sa, long ld_sa,
                                         const void* b, const float* sb,
                                         void* d, const int* m_indices,
                                         int m_total, int n, int k, int num_groups,
                                         int a_fmt, int b_fmt, void* stream);
int dg_m_grouped_gemm_fp8_masked_fmt(const void* a, const float* sa, long ld_sa,
                                     const void* b, const float* sb,
                                     void* d, const int* masked_m,
                                     int num_groups, int max_m, int n, int k,
                                     int a_fmt, int b_fmt, void* stream);

/* Input element types of the casts below. */
enum { DG_DTYPE_F32 = 0, DG_DTYPE_BF16 = 1 };

/* FP8 cast with per-1x128 scales -- the "prior kernel" the README's usage paragraph
 * asks for: it produces A and sA exactly as dg_gemm_fp8_nt and the grouped calls read
 * them (sA MN-major, i.e. the transposed LHS scales the README requires).
 *   x  [rows][ldx]   fp32 or bf16 (x_dtype), device       q  [rows][ldq]  E4M3 bytes
 *   sa [k/128][ld_sa] fp32, sa[kb * ld_sa + row]
 * Per (row, 128-K block): amax = max |x| (NaN entries ignored), scale = fp32(amax/448)
 * (1 if amax == 0), q = E4M3 RNE of fp32(x / scale), saturating at +-448, NaN -> 0x7F.
 * Requires k % 128 == 0 (DG_ERR_UNSUPPORTED), x 16-byte aligned with ldx a multiple of
 * 16 bytes / element size, q 8-byte aligned with ldq % 8 == 0, ld_sa >= rows (else
 * DG_ERR_INVALID_ARG), and sa 16-byte aligned with ld_sa a multiple of 4 -- the sA the
 * GEMMs accept; dg_get_aligned_ld_sa gives the smallest such ld_sa (else
 * DG_ERR_MISALIGNED).  Leading dimensions so large that rows * ld * 4 would not fit
 * in 63 bits give DG_ERR_UNSUPPORTED.  rows == 0 is a no-op.  Asynchronous on
 * `stream`; nothing is allocated. */
int dg_quantize_fp8_1x128(const void* x, int x_dtype, long ldx, int rows, int k,
                          void* q, long ldq, float* sa, long ld_sa, void* stream);

/* FP8 cast with per-128x128 scales (the B-side granularity).
 *   x  [rows][ldx] fp32 or bf16       q [rows][ldq] E4M3       sb [ceil(rows/128)][k/128]
 * Same rounding and requirements as dg_quantize_fp8_1x128 (sb needs 4-byte alignment
 * only); a ragged last row block takes its amax over the rows it has. */
int dg_quantize_fp8_128x128(const void* x, int x_dtype, long ldx, int rows, int k,
                            void* q, long ldq, float* sb, void* stream);

/* The two casts with the output format chosen: q_fmt DG_FMT_E4M3 (exactly the
 * calls above) or DG_FMT_E5M2, E5M2 being the blog's other FP8 format (hnwysp.cn
 * DeepGEMM blog, section 2.3).  For E5M2 the scale is fp32(amax / 57344), the
 * codes are E5M2 RNE of fp32(x / scale) saturating at +-57344 (E5M2's largest
 * finite value; never an infinity), NaN -> 0x7F; everything else as above.  An
 * unknown q_fmt is DG_ERR_INVALID_ARG. */
int dg_quantize_fp8_1x128_fmt(const void* x, int x_dtype, long ldx, int rows, int k,
                              void* q, long ldq, float* sa, long ld_sa, int q_fmt, void* stream);
int dg_quantize_fp8_128x128_fmt(const void* x, int x_dtype, long ldx, int rows, int k,
                                void* q, long ldq, float* sb, int q_fmt, void* stream);

/* Leading dimension (in floats) that an MN-major sA of `rows` rows needs: rows rounded
 * up to a multiple of 4, so that every K block's scales start 16-byte aligned (the
 * README's utility get_tma_aligned_size, for the GEMMs here).  rows < 0 gives
 * DG_ERR_INVALID_ARG, rows above LONG_MAX - 3 DG_ERR_UNSUPPORTED.  Host only. */
long dg_get_aligned_ld_sa(long rows);

/* The README's other sA utility (get_col_major_tma_aligned_tensor): turn per-row scales
 * stored row-major into the MN-major layout the GEMMs read.
 *   sa_in  [groups][rows][ld_in]    fp32, device; sa_in[(g*rows + r)*ld_in + kb]
 *   sa_out [groups][kblocks][ld_sa] fp32, device; sa_out[(g*kblocks + kb)*ld_sa + r]
 * (groups = 1 for the dense and contiguous layouts, G for the masked one.)  Columns
 * rows .. ld_sa-1 of sa_out are left as they are.  Requires ld_in >= kblocks and
 * ld_sa >= rows (else DG_ERR_INVALID_ARG), sa_in 4-byte and sa_out 16-byte aligned and
 * ld_sa % 4 == 0 (else DG_ERR_MISALIGNED), rows * ld_in and kblocks * ld_sa below 2^31
 * and groups <= 65535 (else DG_ERR_UNSUPPORTED).  The two buffers must not overlap.
 * rows == 0 or kblocks == 0 is a no-op.  Asynchronous on `stream`. */
int dg_transform_sa_mn_major(const float* sa_in, long ld_in, float* sa_out, long ld_sa,
                             int rows, int kblocks, int groups, void* stream);

/* Check, on the host, the precondition the contiguous layout places on m_indices (a
 * HOST copy of it): m_total a multiple of dg_get_m_alignment(); every entry a group in
 * [0, num_groups) or -1; in each aligned 128-row block, every entry either -1 or the
 * group of the block's first row (so a block whose first row is padding is all
 * padding).  Returns DG_OK, or DG_ERR_INVALID_ARG with *bad_row (if bad_row is not
 * NULL) set to the first offending row (m_total when m_total is not aligned); bad_row
 * is -1 on success.  The GEMM itself never reads m_indices on the host: a block that
 * breaks the rule gets only its first row's group computed and written. */
int dg_check_contiguous_layout(const int* m_indices, int m_total, int num_groups, int* bad_row);

/* Host-only tile planner, exposed for inspection and tests; it touches no device.
 * Among candidate block shapes (block_ms[i], block_ns[j]) with per-shape relative
 * throughput eff[i * n_bn + j] (NULL = all 1), pick the one that minimises
 *     ceil(tiles / slots) * block_m * block_n / eff,
 * tiles = ceil(m / block_m) * ceil(n / block_n), slots = num_units * blocks_per_unit.
 * This is the unaligned-block-size rule of the README's optimisation section
 * (M=256, N=7168 on 132 SMs: 128x128 fills 112 SMs, 128x112 fills 128).
 * Ties go to fewer waves, then to the earlier candidate.  out[0..3] = block_m, block_n, tiles, waves.
 * Returns the index i * n_bn + j of the chosen pair, or DG_ERR_INVALID_ARG. */
int dg_plan_tiles(int m, int n, int num_units, int blocks_per_unit,
                  const int* block_ms, int n_bm, const int* block_ns, int n_bn,
                  const double* eff, int* out);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
