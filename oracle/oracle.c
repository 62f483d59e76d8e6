/*
 * oracle.c -- plain, slow, CPU-only reference for the fine-grained-scaled
 * FP8 E4M3 "NT" GEMM (dense, M-grouped contiguous, M-grouped masked), and for
 * the dense GEMM with E5M2 operands.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP library is
 * checked against.  Only the test suite, the smoke check and the bench's CPU
 * baseline leg may load it.  It shares no code, header, table or constant with
 * the GPU library, and the GPU library never calls it.
 *
 * Sources (the web pages this method is described on):
 *  - "DeepGEMM: clean and efficient FP8 GEMM kernels with fine-grained scaling"
 *    (nipponese.news Japanese translation of the project README):
 *      intro paragraph          -- FP8 GEMM with DeepSeek-V3 fine-grained scaling,
 *                                  two-level (promoted) accumulation;
 *      usage paragraph (NT)     -- LHS [M,K] non-transposed, RHS [N,K] transposed,
 *                                  LHS scales stored transposed; BF16 output;
 *      contiguous-layout para.  -- groups along M only, N and K shared, segments
 *                                  padded to the M-block alignment;
 *      masked-layout paragraph  -- per-group capacity, a mask of valid rows,
 *                                  only the valid part is computed.
 *  - hnwysp.cn DeepGEMM blog, section 4.1 (E4M3 range is about +-448, values
 *    must be scaled into range) and section 4.3 (accumulate in FP32 or better).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - scale granularity: A one fp32 scale per (row, 128-wide K block); B one
 *    fp32 scale per (128-row N block, 128-wide K block);
 *  - sA stored MN-major: sa[kb * ld_sa + m];  sB stored [ceil(N/128)][ceil(K/128)];
 *  - E4M3 is the OCP E4M3FN encoding (max 448, subnormals, NaN = S.1111.111, no inf);
 *  - the exact result is  D[m,n] = sum_kb sA[m,kb]*sB[n/128,kb]*P_kb(m,n) with
 *    P_kb the exact dot product over the K block, evaluated here in fp64 and
 *    rounded once to BF16 (round-to-nearest-even);
 *  - a K that is not a multiple of 128 ends in a short last block whose scale
 *    covers only the remaining columns;
 *  - E5M2 (hnwysp.cn blog section 2.3 lists it beside E4M3; the README's
 *    functions are FP8 x FP8) is the OCP E5M2 encoding (max 57344, subnormals,
 *    infinities, NaN = S.11111.{01,10,11}); either operand may use it, the
 *    scales and the promotion are unchanged.
 *
 * Why fp64 is (nearly) exact here: every E4M3 value is an integer multiple of
 * 2^-9 with magnitude below 2^18 units, so every product is an integer multiple
 * of 2^-18 below 2^36 units and a 128-term block sum stays below 2^43 units --
 * exact in a 53-bit significand in any summation order.  The product of two
 * fp32 scales is exact in fp64.  The only roundings are one multiply and one
 * add per K block (relative 2^-53) and the final BF16 rounding.  With an E5M2
 * operand the block sum can need more than 53 bits; it is formed exactly in
 * 128-bit integers and rounded once to fp64.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_KBLOCK 128

/* ------------------------------------------------------------------------- */
/* E4M3 (OCP E4M3FN) decode, built from the bit fields.                      */
/* Byte layout s.eeee.fff, exponent bias 7.                                  */
/*   e == 15 && f == 7  -> NaN  (0x7F, 0xFF); there is no infinity           */
/*   e == 0             -> subnormal (-1)^s * f * 2^-9                       */
/*   otherwise          -> (-1)^s * (1 + f/8) * 2^(e-7) = (8+f) * 2^(e-10)   */
/* ------------------------------------------------------------------------- */
static double e4m3_value(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, f = b & 7u;
    double mag;
    if (e == 15u && f == 7u) return NAN;
    if (e == 0u) mag = ldexp((double)f, -9);
    else mag = ldexp((double)(8u + f), (int)e - 10);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------------- */
/* E5M2 (OCP), the second FP8 format the hnwysp.cn blog lists for operands   */
/* (section 2.3).  Byte layout s.eeeee.ff, exponent bias 15.                 */
/*   e == 31: f == 0 -> +-infinity, otherwise NaN                            */
/*   e == 0          -> subnormal (-1)^s * f * 2^-16                         */
/*   otherwise       -> (-1)^s * (1 + f/4) * 2^(e-15) = (4+f) * 2^(e-17)     */
/* ------------------------------------------------------------------------- */
static double e5m2_value(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 2) & 31u, f = b & 3u;
    double mag;
    if (e == 31u) mag = f == 0u ? INFINITY : NAN;
    else if (e == 0u) mag = ldexp((double)f, -16);
    else mag = ldexp((double)(4u + f), (int)e - 17);
    return s ? -mag : mag;
}

/* Every finite value of a format is an integer multiple of its smallest
 * subnormal, 2^-SHIFT: MANT[b] = value * 2^SHIFT (E4M3: |MANT| <= 229376,
 * E5M2: |MANT| <= 57344 * 2^16 < 2^32). */
static const int FMT_SHIFT[2] = {9, 16};

static double DEC[256];          /* E4M3 */
static double DEC5[256];         /* E5M2 */
static int64_t MANT[2][256];
static pthread_once_t dec_once = PTHREAD_ONCE_INIT;
static void dec_init(void)
{
    for (unsigned b = 0; b < 256u; ++b) {
        DEC[b] = e4m3_value(b);
        DEC5[b] = e5m2_value(b);
        MANT[0][b] = isfinite(DEC[b]) ? (int64_t)ldexp(DEC[b], FMT_SHIFT[0]) : 0;
        MANT[1][b] = isfinite(DEC5[b]) ? (int64_t)ldexp(DEC5[b], FMT_SHIFT[1]) : 0;
    }
}

void orc_e4m3_decode_table(double out[256])
{
    pthread_once(&dec_once, dec_init);
    memcpy(out, DEC, sizeof(DEC));
}

void orc_e5m2_decode_table(double out[256])
{
    pthread_once(&dec_once, dec_init);
    memcpy(out, DEC5, sizeof(DEC5));
}

/* ------------------------------------------------------------------------- */
/* E4M3 encode: round to nearest, ties to even mantissa, saturating to       */
/* +-448 (the format's largest finite value, hnwysp.cn blog section 4.1).    */
/* NaN in gives 0x7F.  The sign of zero is kept.                             */
/* ------------------------------------------------------------------------- */
uint8_t orc_e4m3_encode(double x)
{
    unsigned sign;
    double a, q, n;
    int e, E;
    if (isnan(x)) return 0x7Fu;
    sign = signbit(x) ? 0x80u : 0u;
    a = fabs(x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0) return (uint8_t)sign;
    frexp(a, &e);               /* a = frac * 2^e, frac in [0.5, 1) */
    E = e - 1;                  /* floor(log2(a)) */
    if (E < -6) E = -6;         /* below the smallest normal the quantum stays 2^-9 */
    q = ldexp(1.0, E - 3);      /* 3 stored mantissa bits */
    n = nearbyint(a / q);       /* exact division by a power of two; RNE (default mode) */
    if (n < 8.0) return (uint8_t)(sign | (unsigned)n);          /* subnormal (E == -6) */
    if (n >= 16.0) { n = 8.0; E += 1; }                          /* carry into exponent */
    if (E + 7 > 15 || (E + 7 == 15 && n - 8.0 > 6.0))           /* cannot happen below 448 */
        return (uint8_t)(sign | 0x7Eu);
    return (uint8_t)(sign | ((unsigned)(E + 7) << 3) | (unsigned)(n - 8.0));
}

/* ------------------------------------------------------------------------- */
/* E5M2 encode: round to nearest, ties to even mantissa, saturating to       */
/* +-57344 (the format's largest finite value; the same reading as for       */
/* E4M3: a scaled value never lands on an infinity).  NaN in gives 0x7F.     */
/* Exponent bias 15, 2 stored mantissa bits, subnormal quantum 2^-16.        */
/* ------------------------------------------------------------------------- */
uint8_t orc_e5m2_encode(double x)
{
    unsigned sign;
    double a, q, n;
    int e, E;
    if (isnan(x)) return 0x7Fu;
    sign = signbit(x) ? 0x80u : 0u;
    a = fabs(x);
    if (a >= 57344.0) return (uint8_t)(sign | 0x7Bu);
    if (a == 0.0) return (uint8_t)sign;
    frexp(a, &e);               /* a = frac * 2^e, frac in [0.5, 1) */
    E = e - 1;                  /* floor(log2(a)) */
    if (E < -14) E = -14;       /* below the smallest normal the quantum stays 2^-16 */
    q = ldexp(1.0, E - 2);      /* 2 stored mantissa bits */
    n = nearbyint(a / q);       /* exact division by a power of two; RNE (default mode) */
    if (n < 4.0) return (uint8_t)(sign | (unsigned)n);          /* subnormal (E == -14) */
    if (n >= 8.0) { n = 4.0; E += 1; }                           /* carry into exponent */
    if (E + 15 > 30) return (uint8_t)(sign | 0x7Bu);            /* cannot happen below 57344 */
    return (uint8_t)(sign | ((unsigned)(E + 15) << 2) | (unsigned)(n - 4.0));
}

/* ------------------------------------------------------------------------- */
/* BF16 encode from double: round to nearest, ties to even, one rounding.    */
/* 8 significant bits; below 2^-126 the quantum is fixed at 2^-133           */
/* (subnormals); results of magnitude >= 2^128 after rounding become inf;    */
/* NaN gives the canonical quiet NaN 0x7FC0.                                 */
/* ------------------------------------------------------------------------- */
uint16_t orc_bf16_encode(double x)
{
    unsigned sign;
    double a, q, n;
    int e, E;
    if (isnan(x)) return 0x7FC0u;
    sign = signbit(x) ? 0x8000u : 0u;
    a = fabs(x);
    if (a == 0.0) return (uint16_t)sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    frexp(a, &e);
    E = e - 1;
    if (E < -126) E = -126;
    if (E > 127) return (uint16_t)(sign | 0x7F80u);
    q = ldexp(1.0, E - 7);
    n = nearbyint(a / q);
    if (n < 128.0) return (uint16_t)(sign | (unsigned)n);      /* subnormal (E == -126) */
    if (n >= 256.0) { n = 128.0; E += 1; }
    if (E > 127) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | ((unsigned)(E + 127) << 7) | (unsigned)(n - 128.0));
}

/* ------------------------------------------------------------------------- */
/* Quantisers (input preparation; the pages leave the cast to a prior        */
/* kernel).  scale = fp32(amax / FMAX); q = FP8_RNE(clamp(fp32(x / scale)))  */
/* with amax == 0 giving scale 1, FMAX = 448 for E4M3 (fmt 0) and 57344 for  */
/* E5M2 (fmt 1).  Arithmetic is fp32, as a cast kernel working on fp32 input */
/* would do it.                                                              */
/* ------------------------------------------------------------------------- */
static float block_scale(float amax, int fmt)
{
    volatile float s = amax / (fmt ? 57344.0f : 448.0f);
    return amax == 0.0f ? 1.0f : s;
}

static uint8_t quant_one(float x, float s, int fmt)
{
    volatile float y = x / s;
    return fmt ? orc_e5m2_encode((double)y) : orc_e4m3_encode((double)y);
}

void orc_quantize_rows_1x128_fmt(const float* x, long ldx, int m, int k,
                                 uint8_t* q, long ldq, float* sa, long ld_sa, int fmt);
void orc_quantize_blocks_128x128_fmt(const float* x, long ldx, int n, int k,
                                     uint8_t* q, long ldq, float* sb, int fmt);

/* A-side: one scale per (row, 128-wide K block), stored sa[kb * ld_sa + m]. */
void orc_quantize_rows_1x128(const float* x, long ldx, int m, int k,
                             uint8_t* q, long ldq, float* sa, long ld_sa)
{
    orc_quantize_rows_1x128_fmt(x, ldx, m, k, q, ldq, sa, ld_sa, 0);
}

void orc_quantize_rows_1x128_fmt(const float* x, long ldx, int m, int k,
                                 uint8_t* q, long ldq, float* sa, long ld_sa, int fmt)
{
    int kbn = (k + ORC_KBLOCK - 1) / ORC_KBLOCK;
    for (int i = 0; i < m; ++i) {
        for (int kb = 0; kb < kbn; ++kb) {
            int k0 = kb * ORC_KBLOCK, k1 = k0 + ORC_KBLOCK < k ? k0 + ORC_KBLOCK : k;
            float amax = 0.0f, s;
            for (int kk = k0; kk < k1; ++kk) {
                float v = fabsf(x[(long)i * ldx + kk]);
                if (v > amax) amax = v;
            }
            s = block_scale(amax, fmt);
            sa[(long)kb * ld_sa + i] = s;
            for (int kk = k0; kk < k1; ++kk)
                q[(long)i * ldq + kk] = quant_one(x[(long)i * ldx + kk], s, fmt);
        }
    }
}

/* B-side: one scale per (128-row N block, 128-wide K block), sb[nb * Kb + kb]. */
void orc_quantize_blocks_128x128(const float* x, long ldx, int n, int k,
                                 uint8_t* q, long ldq, float* sb)
{
    orc_quantize_blocks_128x128_fmt(x, ldx, n, k, q, ldq, sb, 0);
}

void orc_quantize_blocks_128x128_fmt(const float* x, long ldx, int n, int k,
                                     uint8_t* q, long ldq, float* sb, int fmt)
{
    int kbn = (k + ORC_KBLOCK - 1) / ORC_KBLOCK;
    int nbn = (n + ORC_KBLOCK - 1) / ORC_KBLOCK;
    for (int nb = 0; nb < nbn; ++nb) {
        int n0 = nb * ORC_KBLOCK, n1 = n0 + ORC_KBLOCK < n ? n0 + ORC_KBLOCK : n;
        for (int kb = 0; kb < kbn; ++kb) {
            int k0 = kb * ORC_KBLOCK, k1 = k0 + ORC_KBLOCK < k ? k0 + ORC_KBLOCK : k;
            float amax = 0.0f, s;
            for (int r = n0; r < n1; ++r)
                for (int kk = k0; kk < k1; ++kk) {
                    float v = fabsf(x[(long)r * ldx + kk]);
                    if (v > amax) amax = v;
                }
            s = block_scale(amax, fmt);
            sb[(long)nb * kbn + kb] = s;
            for (int r = n0; r < n1; ++r)
                for (int kk = k0; kk < k1; ++kk)
                    q[(long)r * ldq + kk] = quant_one(x[(long)r * ldx + kk], s, fmt);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Exact block dot product P_kb = sum_{k in block} dec(a_k) * dec(b_k).      */
/* ------------------------------------------------------------------------- */
double orc_block_dot(const uint8_t* a, const uint8_t* b, int len)
{
    double p = 0.0;
    pthread_once(&dec_once, dec_init);
    for (int t = 0; t < len; ++t) p += DEC[a[t]] * DEC[b[t]];
    return p;
}

/* The same block dot product with each operand in its own format (0 = E4M3,
 * 1 = E5M2).  With E5M2 a 128-term sum no longer fits a 53-bit significand, so
 * the products of the integer forms are summed exactly in 128-bit integers and
 * the sum is rounded once to fp64 (then scaled by a power of two, exact).  A
 * block holding an infinity or a NaN is summed in fp64 instead, which gives
 * the IEEE result. */
double orc_block_dot_fmt(const uint8_t* a, const uint8_t* b, int len, int fa, int fb)
{
    const double* da;
    const double* db;
    __int128 sum = 0;
    int finite = 1;
    pthread_once(&dec_once, dec_init);
    da = fa ? DEC5 : DEC;
    db = fb ? DEC5 : DEC;
    for (int t = 0; t < len; ++t) finite &= isfinite(da[a[t]]) && isfinite(db[b[t]]);
    if (!finite) {
        double p = 0.0;
        for (int t = 0; t < len; ++t) p += da[a[t]] * db[b[t]];
        return p;
    }
    for (int t = 0; t < len; ++t) sum += (__int128)MANT[fa][a[t]] * (__int128)MANT[fb][b[t]];
    return ldexp((double)sum, -(FMT_SHIFT[fa] + FMT_SHIFT[fb]));
}

/* One output element of the method (all layouts reduce to this):           */
/*   acc = sum_kb (sA[kb] * sB[kb]) * P_kb,  kb ascending, fp64.             */
static double scaled_row_col(const uint8_t* arow, const float* sa_col, long ld_sa,
                             const uint8_t* brow, const float* sb_row, int k, int fa, int fb)
{
    int kbn = (k + ORC_KBLOCK - 1) / ORC_KBLOCK;
    double acc = 0.0;
    for (int kb = 0; kb < kbn; ++kb) {
        int k0 = kb * ORC_KBLOCK, len = k - k0 < ORC_KBLOCK ? k - k0 : ORC_KBLOCK;
        double p = (fa || fb) ? orc_block_dot_fmt(arow + k0, brow + k0, len, fa, fb)
                              : orc_block_dot(arow + k0, brow + k0, len);
        double s = (double)sa_col[(long)kb * ld_sa] * (double)sb_row[kb];
        acc += s * p;
    }
    return acc;
}

/* ------------------------------------------------------------------------- */
/* Row-parallel driver.                                                      */
/* ------------------------------------------------------------------------- */
typedef struct {
    /* problem */
    const uint8_t* a; long lda;
    const float* sa; long ld_sa; long sa_group_stride;
    const uint8_t* b; long ldb; long b_group_stride;
    const float* sb; long sb_group_stride;
    uint16_t* d; long ldd;
    int m, n, k;
    int layout;               /* 0 dense, 1 contiguous, 2 masked */
    const int* m_indices;     /* contiguous */
    const int* masked_m;      /* masked */
    int max_m;                /* masked: rows per group */
    double* acc_out;          /* optional fp64 result (same indexing as d), may be NULL */
    int a_fmt, b_fmt;         /* operand formats: 0 E4M3, 1 E5M2 */
    /* work split */
    int nthreads, tid;
} orc_job;

static void do_row(const orc_job* J, long row)
{
    int g = 0;
    long local = row;               /* row inside its group (masked) */
    const uint8_t* arow = J->a + row * J->lda;
    const float* sa_col;
    const uint8_t* bg;
    const float* sbg;
    int kbn = (J->k + ORC_KBLOCK - 1) / ORC_KBLOCK;

    if (J->layout == 1) {
        g = J->m_indices[row];
        if (g < 0) return;           /* padding row: not computed, left untouched */
        sa_col = J->sa + row;
    } else if (J->layout == 2) {
        int mm;
        g = (int)(row / J->max_m);
        local = row % J->max_m;
        mm = J->masked_m[g];
        if (mm < 0) mm = 0;
        if (mm > J->max_m) mm = J->max_m;
        if (local >= mm) return;     /* masked row: never written */
        sa_col = J->sa + (long)g * J->sa_group_stride + local;
    } else {
        sa_col = J->sa + row;
    }
    bg = J->b + (long)g * J->b_group_stride;
    sbg = J->sb + (long)g * J->sb_group_stride;
    for (int j = 0; j < J->n; ++j) {
        double acc = scaled_row_col(arow, sa_col, J->ld_sa, bg + (long)j * J->ldb,
                                    sbg + (long)(j / ORC_KBLOCK) * kbn, J->k, J->a_fmt, J->b_fmt);
        J->d[row * J->ldd + j] = orc_bf16_encode(acc);
        if (J->acc_out) J->acc_out[row * J->ldd + j] = acc;
    }
}

static void* worker(void* arg)
{
    const orc_job* J = (const orc_job*)arg;
    for (long row = J->tid; row < J->m; row += J->nthreads) do_row(J, row);
    return NULL;
}

int orc_available_cores(void)
{
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof(set), &set) != 0) return 1;
    return CPU_COUNT(&set) > 0 ? CPU_COUNT(&set) : 1;
}

static int run_rows(orc_job base, int nthreads)
{
    pthread_t th[256];
    orc_job jobs[256];
    int started = 0;
    pthread_once(&dec_once, dec_init);
    if (nthreads <= 0) nthreads = orc_available_cores();
    if (nthreads > 256) nthreads = 256;
    if (nthreads > base.m && base.m > 0) nthreads = base.m;
    if (base.m <= 0 || base.n <= 0) return 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].nthreads = nthreads;
        jobs[t].tid = t;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) break;
        started = t;
    }
    worker(&jobs[0]);
    for (int t = started + 1; t < nthreads; ++t) worker(&jobs[t]); /* threads that failed to start */
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    return nthreads;
}

/* Dense NT GEMM.  A [m][lda] E4M3, sa [Kb][ld_sa], B [n][ldb] E4M3,
 * sb [ceil(n/128)][Kb], D [m][ldd] BF16 bits.  Returns threads used. */
int orc_gemm_fp8_nt(const uint8_t* a, long lda, const float* sa, long ld_sa,
                    const uint8_t* b, long ldb, const float* sb,
                    uint16_t* d, long ldd, double* acc_out,
                    int m, int n, int k, int nthreads)
{
    orc_job J;
    memset(&J, 0, sizeof(J));
    J.a = a; J.lda = lda; J.sa = sa; J.ld_sa = ld_sa;
    J.b = b; J.ldb = ldb; J.sb = sb; J.d = d; J.ldd = ldd; J.acc_out = acc_out;
    J.m = m; J.n = n; J.k = k; J.layout = 0;
    return run_rows(J, nthreads);
}

/* Dense NT GEMM with each operand in its own FP8 format (0 E4M3, 1 E5M2);
 * otherwise as orc_gemm_fp8_nt, which it equals for two E4M3 operands. */
int orc_gemm_fp8_nt_fmt(const uint8_t* a, long lda, const float* sa, long ld_sa,
                        const uint8_t* b, long ldb, const float* sb,
                        uint16_t* d, long ldd, double* acc_out,
                        int m, int n, int k, int a_fmt, int b_fmt, int nthreads)
{
    orc_job J;
    memset(&J, 0, sizeof(J));
    J.a = a; J.lda = lda; J.sa = sa; J.ld_sa = ld_sa;
    J.b = b; J.ldb = ldb; J.sb = sb; J.d = d; J.ldd = ldd; J.acc_out = acc_out;
    J.m = m; J.n = n; J.k = k; J.layout = 0;
    J.a_fmt = a_fmt != 0; J.b_fmt = b_fmt != 0;
    return run_rows(J, nthreads);
}

/* M-grouped contiguous: A [m_total][k], sa [Kb][ld_sa], B [G][n][k],
 * sb [G][ceil(n/128)][Kb], D [m_total][n]; m_indices[row] = group or -1.
 * Rows with -1 are not written.  Operand formats as in orc_gemm_fp8_nt_fmt. */
int orc_m_grouped_contiguous_fmt(const uint8_t* a, const float* sa, long ld_sa,
                                 const uint8_t* b, const float* sb,
                                 uint16_t* d, double* acc_out, const int* m_indices,
                                 int m_total, int n, int k, int num_groups,
                                 int a_fmt, int b_fmt, int nthreads)
{
    orc_job J;
    int kbn = (k + ORC_KBLOCK - 1) / ORC_KBLOCK, nbn = (n + ORC_KBLOCK - 1) / ORC_KBLOCK;
    (void)num_groups;
    memset(&J, 0, sizeof(J));
    J.a = a; J.lda = k; J.sa = sa; J.ld_sa = ld_sa;
    J.b = b; J.ldb = k; J.b_group_stride = (long)n * k;
    J.sb = sb; J.sb_group_stride = (long)nbn * kbn;
    J.d = d; J.ldd = n; J.acc_out = acc_out;
    J.m = m_total; J.n = n; J.k = k; J.layout = 1; J.m_indices = m_indices;
    J.a_fmt = a_fmt != 0; J.b_fmt = b_fmt != 0;
    return run_rows(J, nthreads);
}

int orc_m_grouped_contiguous(const uint8_t* a, const float* sa, long ld_sa,
                             const uint8_t* b, const float* sb,
                             uint16_t* d, double* acc_out, const int* m_indices,
                             int m_total, int n, int k, int num_groups, int nthreads)
{
    return orc_m_grouped_contiguous_fmt(a, sa, ld_sa, b, sb, d, acc_out, m_indices, m_total, n, k, num_groups,
                                        0, 0, nthreads);
}

/* M-grouped masked: A [G][max_m][k], sa [G][Kb][ld_sa], B [G][n][k],
 * sb [G][ceil(n/128)][Kb], D [G][max_m][n]; rows >= masked_m[g] (clamped to
 * [0, max_m]) are not written.  Operand formats as in orc_gemm_fp8_nt_fmt. */
int orc_m_grouped_masked_fmt(const uint8_t* a, const float* sa, long ld_sa,
                             const uint8_t* b, const float* sb,
                             uint16_t* d, double* acc_out, const int* masked_m,
                             int num_groups, int max_m, int n, int k,
                             int a_fmt, int b_fmt, int nthreads)
{
    orc_job J;
    int kbn = (k + ORC_KBLOCK - 1) / ORC_KBLOCK, nbn = (n + ORC_KBLOCK - 1) / ORC_KBLOCK;
    memset(&J, 0, sizeof(J));
    J.a = a; J.lda = k; J.sa = sa; J.ld_sa = ld_sa; J.sa_group_stride = (long)kbn * ld_sa;
    J.b = b; J.ldb = k; J.b_group_stride = (long)n * k;
    J.sb = sb; J.sb_group_stride = (long)nbn * kbn;
    J.d = d; J.ldd = n; J.acc_out = acc_out;
    J.m = num_groups * max_m; J.n = n; J.k = k; J.layout = 2;
    J.masked_m = masked_m; J.max_m = max_m;
    J.a_fmt = a_fmt != 0; J.b_fmt = b_fmt != 0;
    return run_rows(J, nthreads);
}

int orc_m_grouped_masked(const uint8_t* a, const float* sa, long ld_sa,
                         const uint8_t* b, const float* sb,
                         uint16_t* d, double* acc_out, const int* masked_m,
                         int num_groups, int max_m, int n, int k, int nthreads)
{
    return orc_m_grouped_masked_fmt(a, sa, ld_sa, b, sb, d, acc_out, masked_m, num_groups, max_m, n, k,
                                    0, 0, nthreads);
}
