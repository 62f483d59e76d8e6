/* block_scale_check.c -- CPU replay of the FP8 casts' block-scale arithmetic.
 *
 * The cast kernels form each block's scale fp32(amax / FMAX) (FMAX = 448 for E4M3,
 * 57344 for E5M2) without a division on their fast path:
 *     r = RN(1 / FMAX)            (a constant)
 *     q = RN(amax * r)
 *     e = fma(-q, FMAX, amax)     (the residual, exact)
 *     s = fma(e, r, q)
 * for FMAX * 2^-125 <= amax <= 2^127 (every other amax takes the IEEE division).  This
 * program replays those steps with IEEE single-precision arithmetic (each operation
 * rounded once, to nearest even, subnormals kept -- what the GPU does) for EVERY fp32
 * value of that range and counts where the result differs from the IEEE quotient
 * amax / FMAX.
 *
 * Usage: block_scale_check FMAX [threads [uncorrected]]
 *   -> prints "checked N mismatches M first X"; exit status 0 when no value differs.
 * "uncorrected" replays q alone (no correction step) over the first 2^24 values of the
 * range, to show that the comparison notices a quotient that is only faithful.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#if !defined(__FMA__)
#error "build with -mfma: the replay needs single-rounding fused multiply-adds"
#endif

static float g_b, g_r;
static int g_uncorrected;
static uint32_t g_lo, g_hi;   /* bit patterns [g_lo, g_hi] */

typedef struct {
    uint32_t lo, hi;
    unsigned long long bad;
    uint32_t first_bad;
} Job;

static float from_bits(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static void* run(void* p) {
    Job* j = (Job*)p;
    const float b = g_b, r = g_r;
    for (uint64_t u = j->lo; u <= j->hi; ++u) {
        const float amax = from_bits((uint32_t)u);
        volatile float q_ = amax * r; /* volatile: one rounded product, never contracted */
        const float q = q_;
        const float e = fmaf(-q, b, amax);
        const float s = g_uncorrected ? q : fmaf(e, r, q);
        const float ref = amax / b;
        if (to_bits(s) != to_bits(ref)) {
            if (j->bad == 0) j->first_bad = (uint32_t)u;
            ++j->bad;
        }
    }
    return NULL;
}

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s FMAX [threads]\n", argv[0]);
        return 2;
    }
    g_b = (float)atof(argv[1]);
    int nt = argc > 2 ? atoi(argv[2]) : 8;
    if (nt < 1) nt = 1;
    if (nt > 64) nt = 64;
    g_r = 1.0f / g_b;
    g_lo = to_bits(g_b * 0x1p-125f);
    g_hi = to_bits(0x1p127f);
    g_uncorrected = argc > 3 && strcmp(argv[3], "uncorrected") == 0;
    if (g_uncorrected) g_hi = g_lo + (1u << 24) - 1;
    Job jobs[64];
    pthread_t th[64];
    const uint64_t total = (uint64_t)g_hi - g_lo + 1;
    for (int t = 0; t < nt; ++t) {
        jobs[t].lo = (uint32_t)(g_lo + total * t / nt);
        jobs[t].hi = (uint32_t)(g_lo + total * (t + 1) / nt - 1);
        jobs[t].bad = 0;
        jobs[t].first_bad = 0;
        pthread_create(&th[t], NULL, run, &jobs[t]);
    }
    unsigned long long bad = 0;
    uint32_t first = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad && !bad) first = jobs[t].first_bad;
        bad += jobs[t].bad;
    }
    printf("checked %llu mismatches %llu first 0x%08x\n", (unsigned long long)total, bad, first);
    return bad == 0 ? 0 : 1;
}
