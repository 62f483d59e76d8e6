// dg_host_check.cpp -- drives libdg.so's C ABI (dg_api.cpp linked with dg_host_stub.cpp,
// no GPU) through validation, planning and the host helpers, for the sanitizer build:
// every call must return the documented status and plan the documented launch, and
// AddressSanitizer / UndefinedBehaviorSanitizer must report nothing.
// Prints one line per failed check; exit status = number of failures.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <thread>
#include <vector>

#include "../../fp8_block_scaled_e4m3_amd/csrc/dg_internal.h"
#include "../../include/dg.h"
#include "../../include/dg_tuning.h"

namespace dg {
extern GemmParams g_last_params;
extern int g_last_grid, g_last_config, g_launches, g_aux_launches;
}  // namespace dg

static int g_fail = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);    \
            ++g_fail;                                                   \
        }                                                               \
    } while (0)

// fake device pointers: aligned addresses that are never dereferenced on the host
static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
static const float* F(uintptr_t x) { return reinterpret_cast<const float*>(x); }
static const int* I(uintptr_t x) { return reinterpret_cast<const int*>(x); }

static int dense(int m, int n, int k, long lda = -1, long ld_sa = -1, long ldb = -1, long ldd = -1,
                 uintptr_t a = 0x1000, uintptr_t sa = 0x2000) {
    if (lda < 0) lda = k;
    if (ldb < 0) ldb = k;
    if (ldd < 0) ldd = n;
    if (ld_sa < 0) ld_sa = ((long)m + 3) / 4 * 4;
    return dg_gemm_fp8_nt(P(a), lda, F(sa), ld_sa, P(0x3000), ldb, F(0x4000), P(0x5000), ldd, m, n, k, nullptr);
}

int main() {
    using dg::g_last_params;
    // ---- dense: the three workload shapes plan as documented
    CHECK(dense(4096, 7168, 7168) == DG_OK);
    CHECK(dg::g_last_config == 5 && g_last_params.num_tiles == 448 && dg::g_last_grid == 256);
    CHECK(g_last_params.tiles_n == 28 && g_last_params.kblocks == 56 && g_last_params.xcd_remap == 1);
    CHECK(dense(256, 7168, 2048) == DG_OK);
    CHECK(dg::g_last_config == 3 && g_last_params.num_tiles == 256 && dg::g_last_grid == 256);
    CHECK(dense(128, 128, 512) == DG_OK);
    CHECK(g_last_params.num_tiles >= 1 && dg::g_last_grid == g_last_params.num_tiles);
    // small M at K = 7168: 64x64 tiles fill more CUs than 64x112 in the same single round, and
    // with fewer tiles than CUs and a long K the configuration with two K groups of waves
    CHECK(dense(64, 4096, 7168) == DG_OK);
    CHECK(dg::g_last_config == 7 && g_last_params.num_tiles == 64 && dg::g_last_grid == 64);   // K groups
    // ---- dense validation, nothing launched on failure
    const int before = dg::g_launches;
    CHECK(dense(128, 128, 200) == DG_ERR_UNSUPPORTED);                // K % 128
    CHECK(dense(128, 120, 512) == DG_ERR_UNSUPPORTED);                // N % 16
    CHECK(dense(128, 128, 512, 520) == DG_ERR_MISALIGNED);            // lda % 16
    CHECK(dense(128, 128, 512, -1, 130) == DG_ERR_MISALIGNED);        // ld_sa % 4
    CHECK(dense(128, 128, 512, -1, 124) == DG_ERR_INVALID_ARG);       // ld_sa < m
    CHECK(dense(128, 128, 512, 256) == DG_ERR_INVALID_ARG);           // lda < k
    CHECK(dense(128, 128, 512, -1, -1, -1, 100) == DG_ERR_INVALID_ARG);   // ldd < n
    CHECK(dense(128, 128, 512, -1, -1, -1, -1, 0x1008) == DG_ERR_MISALIGNED);
    CHECK(dense(-1, 128, 512) == DG_ERR_INVALID_ARG);
    CHECK(dense(0, 128, 512) == DG_OK);                               // empty: no launch
    CHECK(dense(INT_MAX, 128, 512, 1L << 40, -1) == DG_ERR_UNSUPPORTED);  // 32-bit offsets
    CHECK(dense(1 << 20, 1 << 20, 1 << 30) == DG_ERR_UNSUPPORTED);
    CHECK(dense(128, 128, 512, LONG_MAX - 15) == DG_ERR_UNSUPPORTED);         // no overflow in the checks
    CHECK(dense(128, 128, 512, -1, LONG_MAX - 3) == DG_ERR_UNSUPPORTED);
    CHECK(dense(128, 128, 512, -1, -1, LONG_MAX - 15) == DG_ERR_UNSUPPORTED);
    CHECK(dense(128, 128, 512, -1, -1, -1, LONG_MAX - 7) == DG_ERR_UNSUPPORTED);
    CHECK(dg_gemm_fp8_nt_fmt(P(0x1000), 512, F(0x2000), 128, P(0x3000), 512, F(0x4000), P(0x5000), 128, 128, 128,
                             512, 2, 0, nullptr) == DG_ERR_INVALID_ARG);
    CHECK(dg::g_launches == before);
    // ---- E5M2 operands: a configuration that carries them
    CHECK(dg_gemm_fp8_nt_fmt(P(0x1000), 7168, F(0x2000), 4096, P(0x3000), 7168, F(0x4000), P(0x5000), 7168, 4096,
                             7168, 7168, DG_FMT_E5M2, DG_FMT_E4M3, nullptr) == DG_OK);
    CHECK(g_last_params.fmt == 1);

    // ---- contiguous: the Zipf workload (m_total 33280) and validation
    CHECK(dg_m_grouped_gemm_fp8_contiguous(P(0x1000), F(0x2000), 33280, P(0x3000), F(0x4000), P(0x5000), I(0x6000),
                                           33280, 4096, 7168, 8, nullptr) == DG_OK);
    CHECK(dg::g_last_config == 13 && g_last_params.num_tiles == 130 * 16 && g_last_params.num_groups == 8);
    CHECK(dg_m_grouped_gemm_fp8_contiguous(P(0x1000), F(0x2000), 33280, P(0x3000), F(0x4000), P(0x5000), I(0x6000),
                                           33200, 4096, 7168, 8, nullptr) == DG_ERR_INVALID_ARG);
    CHECK(dg_m_grouped_gemm_fp8_contiguous(P(0x1000), F(0x2000), 33280, P(0x3000), F(0x4000), P(0x5000), I(0x6002),
                                           33280, 4096, 7168, 8, nullptr) == DG_ERR_MISALIGNED);
    CHECK(dg_m_grouped_gemm_fp8_contiguous(P(0x1000), F(0x2000), 33280, P(0x3000), F(0x4000), P(0x5000), I(0x6000),
                                           33280, 4096, 7168, 0, nullptr) == DG_ERR_INVALID_ARG);

    // ---- masked: the decode workload, group limits, CU caps
    CHECK(dg_m_grouped_gemm_fp8_masked(P(0x1000), F(0x2000), 256, P(0x3000), F(0x4000), P(0x5000), I(0x6000), 16,
                                       256, 4096, 7168, nullptr) == DG_OK);
    CHECK(dg::g_last_config == 24 && g_last_params.num_tiles == 256 && dg::g_last_grid == 256);
    CHECK(dg_m_grouped_gemm_fp8_masked(P(0x1000), F(0x2000), 256, P(0x3000), F(0x4000), P(0x5000), I(0x6000), 1025,
                                       256, 4096, 7168, nullptr) == DG_ERR_UNSUPPORTED);
    CHECK(dg_set_num_cus(192) == DG_OK);
    CHECK(dg_get_num_cus() == 192);
    CHECK(dg_m_grouped_gemm_fp8_masked(P(0x1000), F(0x2000), 256, P(0x3000), F(0x4000), P(0x5000), I(0x6000), 16,
                                       256, 4096, 7168, nullptr) == DG_OK);
    CHECK(dg::g_last_grid <= 192 && dg::g_last_config == 20);
    // capacity of at most 128 rows: the 128x256 tile (each B tile streamed once, half the A re-reads of 128x128)
    CHECK(dg_set_num_cus(0) == DG_OK);
    CHECK(dg_m_grouped_gemm_fp8_masked(P(0x1000), F(0x2000), 128, P(0x3000), F(0x4000), P(0x5000), I(0x6000), 8,
                                       128, 7168, 2048, nullptr) == DG_OK);
    CHECK(dg::g_last_config == 23 && g_last_params.num_tiles == 8 * 28);
    CHECK(dg_set_num_cus(3) == DG_OK);
    CHECK(dense(4096, 7168, 7168) == DG_OK && dg::g_last_grid == 3 && g_last_params.xcd_remap == 0);
    CHECK(dg_set_num_cus(0) == DG_OK && dg_get_num_cus() == 256);

    // ---- describe / plan / config pinning (per thread)
    int out[8] = {0};
    CHECK(dg_describe_launch(0, 4096, 7168, 7168, 1, 256, out) == DG_OK);
    CHECK(out[0] == 256 && out[1] == 256 && out[3] == 448 && out[4] == 256 && out[5] == 5 && out[7] == 56);
    CHECK(dg_describe_launch(3, 4096, 7168, 7168, 1, 256, out) == DG_ERR_INVALID_ARG);
    const int bms[2] = {128, 128}, bns[2] = {128, 112};
    int po[4] = {0};
    CHECK(dg_plan_tiles(256, 7168, 132, 1, bms, 1, bns, 2, nullptr, po) == 1);
    CHECK(po[0] == 128 && po[1] == 112 && po[2] == 128 && po[3] == 1);
    CHECK(dg_set_kernel_config(0) == DG_OK);
    CHECK(dense(4096, 7168, 7168) == DG_OK && dg::g_last_config == 0);
    int other_thread_config = -1;
    std::thread t([&] {
        dense(4096, 7168, 7168);
        other_thread_config = dg::g_last_config;
    });
    t.join();
    CHECK(other_thread_config == 5);                                   // the pin is this thread's only
    CHECK(dg_set_kernel_config(999) == DG_ERR_INVALID_ARG);
    CHECK(dg_set_kernel_config(-1) == DG_OK);
    CHECK(dense(4096, 7168, 7168) == DG_OK && dg::g_last_config == 5);
    int info[8];
    int ninfo = 0;
    while (dg_kernel_config_info(ninfo, info) == DG_OK) ++ninfo;
    CHECK(ninfo == 17);

    // ---- casts and the sA helpers
    const int aux = dg::g_aux_launches;
    CHECK(dg_quantize_fp8_1x128(P(0x1000), DG_DTYPE_F32, 7168, 4096, 7168, P(0x2000), 7168, (float*)P(0x3000), 4096,
                                nullptr) == DG_OK);
    CHECK(dg_quantize_fp8_1x128(P(0x1000), DG_DTYPE_F32, 7168, 4096, 7168, P(0x2000), 7168, (float*)P(0x3000), 4098,
                                nullptr) == DG_ERR_MISALIGNED);
    CHECK(dg_quantize_fp8_128x128(P(0x1000), DG_DTYPE_BF16, 7168, 7168, 7168, P(0x2000), 7168, (float*)P(0x3004),
                                  nullptr) == DG_OK);
    CHECK(dg_quantize_fp8_1x128(P(0x1000), DG_DTYPE_F32, LONG_MAX - 3, 4, 256, P(0x2000), 256, (float*)P(0x3000), 4,
                                nullptr) != DG_OK);
    CHECK(dg_quantize_fp8_128x128(P(0x1000), DG_DTYPE_BF16, LONG_MAX - 7, 4, 256, P(0x2000), LONG_MAX - 7,
                                  (float*)P(0x3000), nullptr) != DG_OK);
    CHECK(dg_get_aligned_ld_sa(4097) == 4100 && dg_get_aligned_ld_sa(-5) == DG_ERR_INVALID_ARG);
    CHECK(dg_get_aligned_ld_sa(LONG_MAX) == DG_ERR_UNSUPPORTED);
    CHECK(dg_transform_sa_mn_major(F(0x1004), LONG_MAX, (float*)P(0x2000), 4100, 4097, 56, 1, nullptr) ==
          DG_ERR_UNSUPPORTED);
    CHECK(dg_transform_sa_mn_major(F(0x1004), 56, (float*)P(0x2000), 4100, 4097, 56, 1, nullptr) == DG_OK);
    CHECK(dg_transform_sa_mn_major(F(0x1004), 56, (float*)P(0x2000), 4100, 4097, 56, 0, nullptr) ==
          DG_ERR_INVALID_ARG);
    CHECK(dg::g_aux_launches == aux + 3);

    // ---- contiguous layout checker on host arrays of exactly m_total entries
    std::vector<int> mi(384, -1);
    for (int r = 0; r < 130; ++r) mi[r] = 0;
    for (int r = 256; r < 300; ++r) mi[r] = 1;
    int bad = 0;
    CHECK(dg_check_contiguous_layout(mi.data(), (int)mi.size(), 2, &bad) == DG_OK && bad == -1);
    mi[200] = 1;
    CHECK(dg_check_contiguous_layout(mi.data(), (int)mi.size(), 2, &bad) == DG_ERR_INVALID_ARG && bad == 200);
    mi[200] = -1;
    CHECK(dg_check_contiguous_layout(mi.data(), 300, 2, &bad) == DG_ERR_INVALID_ARG && bad == 300);
    CHECK(dg_check_contiguous_layout(nullptr, 0, 1, nullptr) == DG_OK);
    CHECK(dg_check_contiguous_layout(nullptr, 128, 1, &bad) == DG_ERR_INVALID_ARG);

    std::printf("%d failures\n", g_fail);
    return g_fail;
}
