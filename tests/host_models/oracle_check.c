/* oracle_check.c -- drives every exported function of oracle/oracle.c on small,
 * edge-heavy inputs for the sanitizer build (AddressSanitizer and
 * UndefinedBehaviorSanitizer must report nothing) and checks a few closed forms on the
 * way: E4M3 / E5M2 extremes, the identity GEMM, untouched masked and padding rows,
 * and identical results on one and several threads.
 * Prints one line per failed check; exit status = number of failures. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_e4m3_decode_table(double out[256]);
void orc_e5m2_decode_table(double out[256]);
uint8_t orc_e4m3_encode(double x);
uint8_t orc_e5m2_encode(double x);
uint16_t orc_bf16_encode(double x);
void orc_quantize_rows_1x128_fmt(const float* x, long ldx, int m, int k, uint8_t* q, long ldq, float* sa,
                                 long ld_sa, int fmt);
void orc_quantize_blocks_128x128_fmt(const float* x, long ldx, int n, int k, uint8_t* q, long ldq, float* sb,
                                     int fmt);
double orc_block_dot(const uint8_t* a, const uint8_t* b, int len);
double orc_block_dot_fmt(const uint8_t* a, const uint8_t* b, int len, int fa, int fb);
int orc_available_cores(void);
int orc_gemm_fp8_nt_fmt(const uint8_t* a, long lda, const float* sa, long ld_sa, const uint8_t* b, long ldb,
                        const float* sb, uint16_t* d, long ldd, double* acc_out, int m, int n, int k, int a_fmt,
                        int b_fmt, int nthreads);
int orc_m_grouped_contiguous_fmt(const uint8_t* a, const float* sa, long ld_sa, const uint8_t* b, const float* sb,
                                 uint16_t* d, double* acc_out, const int* m_indices, int m_total, int n, int k,
                                 int num_groups, int a_fmt, int b_fmt, int nthreads);
int orc_m_grouped_masked_fmt(const uint8_t* a, const float* sa, long ld_sa, const uint8_t* b, const float* sb,
                             uint16_t* d, double* acc_out, const int* masked_m, int num_groups, int max_m, int n,
                             int k, int a_fmt, int b_fmt, int nthreads);

static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);         \
            ++fails;                                                    \
        }                                                               \
    } while (0)

static uint32_t lcg = 12345u;
static uint32_t rnd(void) {
    lcg = lcg * 1664525u + 1013904223u;
    return lcg >> 8;
}

int main(void) {
    double t4[256], t5[256];
    orc_e4m3_decode_table(t4);
    orc_e5m2_decode_table(t5);
    CHECK(t4[0x7E] == 448.0 && isnan(t4[0x7F]) && t4[0x01] == ldexp(1.0, -9));
    CHECK(t5[0x7B] == 57344.0 && isinf(t5[0x7C]) && t5[0x01] == ldexp(1.0, -16));
    const double edges[] = {0.0, -0.0, 1e-300, -1e-300, 1e300, -1e300, INFINITY, -INFINITY, NAN, 448.0, 464.0,
                            ldexp(1.0, -10), 3 * ldexp(1.0, -10), 57344.0, 61440.0, 1e-45, 3.4e38};
    for (size_t i = 0; i < sizeof(edges) / sizeof(edges[0]); ++i) {
        (void)orc_e4m3_encode(edges[i]);
        (void)orc_e5m2_encode(edges[i]);
        (void)orc_bf16_encode(edges[i]);
    }
    CHECK(orc_e4m3_encode(1e300) == 0x7E && orc_e4m3_encode(-0.0) == 0x80 && orc_e4m3_encode(NAN) == 0x7F);
    CHECK(orc_bf16_encode(1e300) == 0x7F80 && orc_bf16_encode(NAN) == 0x7FC0);

    /* quantisers over ragged shapes with zero, NaN, inf, huge and tiny blocks */
    const int m = 131, k = 384, kb = 3;
    float* x = malloc(sizeof(float) * m * k);
    for (int i = 0; i < m * k; ++i) x[i] = ((int)(rnd() % 2001) - 1000) * 0.01f;
    for (int c = 0; c < 128; ++c) x[c] = 0.0f;
    x[1 * k + 3] = NAN;
    x[2 * k + 200] = INFINITY;
    x[3 * k + 5] = 3e38f;
    x[4 * k + 9] = 1e-44f;
    uint8_t* q = malloc((size_t)m * k);
    float* sa = malloc(sizeof(float) * kb * 132);
    float* sb = malloc(sizeof(float) * 2 * kb);
    for (int fmt = 0; fmt < 2; ++fmt) {
        orc_quantize_rows_1x128_fmt(x, k, m, k, q, k, sa, 132, fmt);
        orc_quantize_blocks_128x128_fmt(x, k, m, k, q, k, sb, fmt);
    }
    CHECK(sa[0] == 1.0f);                                   /* all-zero block: scale 1 */

    /* block dot products: every format pair, all byte values */
    uint8_t ab[256], bb[256];
    for (int i = 0; i < 256; ++i) {
        ab[i] = (uint8_t)i;
        bb[i] = (uint8_t)(255 - i);
    }
    for (int fa = 0; fa < 2; ++fa)
        for (int fb = 0; fb < 2; ++fb) (void)orc_block_dot_fmt(ab, bb, 256, fa, fb);
    (void)orc_block_dot(ab, ab, 128);

    /* identity: A = 1.0 (0x38) on the diagonal, sa = 1 -> D[i][j] = bf16(sB * B[j][i]) */
    const int n = 144, kk = 128;
    uint8_t* a = calloc((size_t)128 * kk, 1);
    uint8_t* b = malloc((size_t)n * kk);
    for (int i = 0; i < 128; ++i) a[i * kk + i] = 0x38;
    for (int i = 0; i < n * kk; ++i) {
        b[i] = (uint8_t)(rnd() & 0xFF);
        if ((b[i] & 0x7F) == 0x7F) b[i] = 0x30;               /* no NaN codes */
    }
    float sa1[128], sb1[2] = {0.5f, 2.0f};
    for (int i = 0; i < 128; ++i) sa1[i] = 1.0f;
    uint16_t* d1 = malloc(sizeof(uint16_t) * 128 * n);
    uint16_t* d4 = malloc(sizeof(uint16_t) * 128 * n);
    double* acc = malloc(sizeof(double) * 128 * n);
    orc_gemm_fp8_nt_fmt(a, kk, sa1, 128, b, kk, sb1, d1, n, acc, 128, n, kk, 0, 0, 1);
    orc_gemm_fp8_nt_fmt(a, kk, sa1, 128, b, kk, sb1, d4, n, NULL, 128, n, kk, 0, 0, 4);
    CHECK(memcmp(d1, d4, sizeof(uint16_t) * 128 * n) == 0);
    int ok = 1;
    for (int i = 0; i < 128; ++i)
        for (int j = 0; j < n; ++j) ok &= acc[i * n + j] == sb1[j / 128] * t4[b[j * kk + i]];
    CHECK(ok);

    /* contiguous: padding rows keep d_init; masked: rows >= masked_m (clamped) keep it */
    int mi[256];
    for (int i = 0; i < 256; ++i) mi[i] = i < 100 ? 0 : (i >= 128 && i < 140 ? 1 : -1);
    uint8_t* ag = malloc((size_t)256 * kk);
    for (int i = 0; i < 256 * kk; ++i) ag[i] = (uint8_t)(rnd() % 0x7E);
    uint8_t* bg = malloc((size_t)2 * n * kk);
    for (int i = 0; i < 2 * n * kk; ++i) bg[i] = (uint8_t)(rnd() % 0x7E);
    float sag[2 * 256], sbg[2 * 2];
    for (int i = 0; i < 2 * 256; ++i) sag[i] = 0.25f;
    for (int i = 0; i < 4; ++i) sbg[i] = 1.5f;
    uint16_t* dg = malloc(sizeof(uint16_t) * 256 * n);
    for (int i = 0; i < 256 * n; ++i) dg[i] = 0x7FE5;
    orc_m_grouped_contiguous_fmt(ag, sag, 256, bg, sbg, dg, NULL, mi, 256, n, kk, 2, 0, 0, 3);
    int untouched = 1;
    for (int i = 0; i < 256; ++i)
        if (mi[i] < 0)
            for (int j = 0; j < n; ++j) untouched &= dg[i * n + j] == 0x7FE5;
    CHECK(untouched);
    const int mm[2] = {-4, 500};
    for (int i = 0; i < 256 * n; ++i) dg[i] = 0x7FE5;
    orc_m_grouped_masked_fmt(ag, sag, 128, bg, sbg, dg, NULL, mm, 2, 128, n, kk, 1, 1, 2);
    untouched = 1;
    for (int j = 0; j < 128 * n; ++j) untouched &= dg[j] == 0x7FE5;        /* group 0: count < 0 -> 0 */
    CHECK(untouched);
    CHECK(orc_available_cores() >= 1);

    free(x); free(q); free(sa); free(sb); free(a); free(b); free(d1); free(d4); free(acc);
    free(ag); free(bg); free(dg);
    printf("%d failures\n", fails);
    return fails;
}
