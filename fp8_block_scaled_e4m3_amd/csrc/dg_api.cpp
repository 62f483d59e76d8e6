// dg_api.cpp -- C ABI of libdg.so: argument validation, tile planning and
// launch of the gfx950 kernels in dg_gemm.hip.  Host code only; it never
// touches device memory (no allocation, copy, read-back or synchronisation), so
// every entry point is asynchronous on the caller's stream and graph-capturable.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/dg.h"
#include "../../include/dg_tuning.h"
#include "dg_internal.h"

namespace {

using dg::GemmParams;
using dg::KernelConfig;

constexpr int kKBlock = 128;
constexpr int kMAlign = 128;           // contiguous-layout segment alignment
constexpr int kMaxMaskedGroups = 1024; // LDS prefix table size in the masked kernel
constexpr int kXcds = 8;
constexpr int kMaxDevices = 64;

std::atomic<int> g_cu_cap{0};
// dg_set_kernel_config: per layout, an index into the config table, or -1.  Per
// thread, so that pinning a configuration never re-plans another thread's calls.
thread_local int g_forced_cfg[3] = {-1, -1, -1};

struct DeviceInfo {
    bool init = false;
    int cus = 0;
    int occ[64] = {0};   // blocks per CU, indexed by position in the config table
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

bool debug_enabled() {
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("DG_DEBUG");
        v = (e && e[0] && e[0] != '0') ? 1 : 0;
    }
    return v == 1;
}

// DG_GROUP_M (tuning): row blocks of the tile raster visited together before
// moving along N; 0 or unset keeps the default of 4.
int group_m_override() {
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("DG_GROUP_M");
        v = e ? std::atoi(e) : 0;
        if (v < 0) v = 0;
    }
    return v;
}

// Returns nullptr when no device is usable.
const DeviceInfo* device_info(int* status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        *status = DG_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo& d = g_dev[dev];
    if (!d.init) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            *status = DG_ERR_HIP;
            return nullptr;
        }
        int count = 0;
        const KernelConfig* cfgs = dg::kernel_configs(&count);
        for (int i = 0; i < count && i < 64; ++i) {
            int blocks = 0;
            if (cfgs[i].occupancy(&blocks) != hipSuccess || blocks <= 0) {
                (void)hipGetLastError();
                blocks = 1;
            }
            d.occ[i] = blocks;
        }
        d.cus = cus;
        d.init = true;
    }
    *status = DG_OK;
    return &d;
}

int effective_cus(int device_cus) {
    const int cap = g_cu_cap.load();
    return (cap > 0 && cap < device_cus) ? cap : device_cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_fmt(int f) { return f == DG_FMT_E4M3 || f == DG_FMT_E5M2; }

// K/128 of the shape instance (N and K fixed at compile time) a launch of config c
// uses, 0 for the generic one (the selection the config's launcher makes: the call's N
// and K/128 listed in kSpecShapes for the config's layout, any operand format)
int specialised_kblocks(const KernelConfig& c, const GemmParams& p) {
    if (!c.shape_specialised) return 0;
    for (const dg::SpecShape& s : dg::kSpecShapes)
        if (s.grouped == (c.layout != dg::kDense) && s.n == p.n && s.kblocks == p.kblocks) return s.kblocks;
    return 0;
}

// The kernels address a tile's operands through 32-bit buffer offsets from the
// tile's first row: up to 256 rows of A or B (row stride lda / ldb bytes) plus the
// K offset, and the A scales of all K blocks (k/128 rows of ld_sa floats).  Sizes
// whose offsets would not fit are refused rather than wrapped.
bool offsets_fit(long lda, long ldb, long ld_sa, int k) {
    const long lim = 0xFFFFFFFFl;
    // (each bound checked before the product it guards, so no product overflows)
    if (lda > lim / 256 || ldb > lim / 256 || ld_sa > lim / 4) return false;
    return 256 * lda + k <= lim && 256 * ldb + k <= lim && (long)(k / kKBlock) * ld_sa * 4 + 4096 <= lim;
}

// GemmParams::fmt: bit 0 = A is E5M2, bit 1 = B is E5M2
int fmt_bits(int a_fmt, int b_fmt) { return (a_fmt == DG_FMT_E5M2 ? 1 : 0) | (b_fmt == DG_FMT_E5M2 ? 2 : 0); }

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// Planner order: the smaller estimated makespan (waves x per-tile work); on a tie
// the plan with fewer waves, i.e. whole waves of larger tiles.
bool better(double cost, long waves, double best_cost, long best_waves) {
    const double tol = 1e-9 * (cost > best_cost ? cost : best_cost);
    if (cost < best_cost - tol) return true;
    if (cost > best_cost + tol) return false;
    return waves < best_waves;
}

// Row tiles per raster group (the tile order visits group_m row tiles across all
// column tiles, then the next group).  With the XCD-aware hand-out each XCD gets
// `chunk` consecutive tiles per round, i.e. a group_m x chunk/group_m block of the
// output, whose A and B rows its L2 fetches once: prefer blocks that never straddle
// two raster groups (group_m * tiles_n a multiple of chunk), then the block with
// the fewest operand rows.  Without the XCD hand-out, 4.
int raster_group_m(int tiles_m, int tiles_n, long chunk, int bm, int bn) {
    if (chunk <= 0) return 4;
    int best = 4;
    long best_rows = 0;
    bool best_whole = false;
    for (int gm = 1; gm <= 16; gm *= 2) {
        if (gm > tiles_m || chunk % gm) continue;
        const bool whole = ((long)gm * tiles_n) % chunk == 0;
        const long rows = (long)gm * bm + chunk / gm * bn;
        if (best_rows == 0 || (whole && !best_whole) || (whole == best_whole && rows < best_rows)) {
            best = gm;
            best_rows = rows;
            best_whole = whole;
        }
    }
    return best;
}

// K groups (two groups of waves splitting a tile's K blocks) shorten each tile's chain
// of block steps but add a second wave per SIMD and a reduction: they paid only where
// the tiles leave CUs idle or just fill them and K is long (64x4096x7168 and
// 128x7168x7168: 11-12% faster), and lost at K = 2048 and with more tiles than CUs.
constexpr int kKGroupMinKBlocks = 32;

// Pick among the compiled configurations of one layout.
int choose_config(int layout, int m, int n, int num_groups, int fmt, int num_units, const DeviceInfo* dev,
                  int max_m_hint, int kblocks) {
    int count = 0;
    const KernelConfig* cfgs = dg::kernel_configs(&count);
    const int forced = g_forced_cfg[layout];
    if (forced >= 0 && forced < count) return (fmt == 0 || cfgs[forced].all_formats) ? forced : -1;
    int best = -1;
    double best_cost = 0.0;
    long best_waves = 0;
    for (int i = 0; i < count; ++i) {
        const KernelConfig& c = cfgs[i];
        if (c.layout != layout || (fmt != 0 && !c.all_formats)) continue;
        // Masked: the whole capacity in one row block when it fits (B is then streamed
        // once per group), else the largest block; among those the cost model below on
        // the upper bound of the tile count (every group full), so that a CU cap that
        // leaves fewer CUs than 256x256 tiles picks narrower tiles.
        if (layout == dg::kMasked && c.bm != (max_m_hint <= 128 ? 128 : 256)) continue;
        // The busiest CU's share: ceil(tiles / CUs) tiles of bm x bn at the shape's
        // relative throughput (workgroups resident together share one CU).
        const long tiles = (layout == dg::kMasked ? num_groups : 1) * ceil_div(m, c.bm) * ceil_div(n, c.bn);
        if (c.wk > 1 && (tiles > num_units || kblocks < kKGroupMinKBlocks)) continue;
        const long waves = ceil_div(tiles, (long)num_units);
        const double cost = (double)waves * c.bm * c.bn / c.eff;
        if (best < 0 || better(cost, waves, best_cost, best_waves)) {
            best = i;
            best_cost = cost;
            best_waves = waves;
        }
    }
    return best;
}

int launch(int layout, GemmParams& p, int m_for_plan, int max_m_hint, hipStream_t stream, int forced_cus,
           int* describe_out) {
    int st = DG_OK;
    const DeviceInfo* dev = nullptr;
    int units = forced_cus;
    if (units <= 0) {
        dev = device_info(&st);
        if (!dev) return st;
        units = effective_cus(dev->cus);
    }
    int count = 0;
    const KernelConfig* cfgs = dg::kernel_configs(&count);
    const int ci = choose_config(layout, m_for_plan, p.n, p.num_groups, p.fmt, units, dev, max_m_hint, p.kblocks);
    if (ci < 0) return DG_ERR_UNSUPPORTED;
    const KernelConfig& c = cfgs[ci];
    const int per_cu = dev ? dev->occ[ci] : 1;

    p.tiles_n = (int)ceil_div(p.n, c.bn);
    p.tiles_m = (int)ceil_div(p.rows, c.bm);
    const long tiles = (long)p.tiles_m * p.tiles_n * (layout == dg::kMasked ? p.num_groups : 1);
    if (tiles > INT_MAX / 2) return DG_ERR_UNSUPPORTED;   // tile indices are 32-bit on the device
    p.num_tiles = (int)tiles;
    long slots = (long)units * per_cu;
    long grid = p.num_tiles < slots ? p.num_tiles : slots;
    if (grid < 1) grid = 1;
    // keep whole rounds of 8 workgroups so the XCD hand-out stays a bijection
    p.xcd_remap = (grid % kXcds == 0) ? 1 : 0;
    p.group_m = group_m_override() > 0 ? group_m_override()
                                       : raster_group_m(p.tiles_m, p.tiles_n, p.xcd_remap ? grid / kXcds : 0, c.bm, c.bn);

    if (describe_out) {
        describe_out[0] = c.bm;
        describe_out[1] = c.bn;
        describe_out[2] = c.wm * c.wn * c.wk;
        describe_out[3] = p.num_tiles;
        describe_out[4] = (int)grid;
        describe_out[5] = c.id;
        describe_out[6] = layout == dg::kMasked ? 0 : p.group_m;
        describe_out[7] = specialised_kblocks(c, p);
        return DG_OK;
    }
    if (debug_enabled())
        std::fprintf(stderr, "[dg] layout=%d rows=%d n=%d k=%d groups=%d cfg=%d (%dx%d, %d waves) tiles=%d grid=%ld units=%d\n",
                     layout, p.rows, p.n, p.k, p.num_groups, c.id, c.bm, c.bn, c.wm * c.wn * c.wk, p.num_tiles, grid, units);
    if (c.launch(p, (int)grid, stream) != hipSuccess) {
        (void)hipGetLastError();
        return DG_ERR_HIP;
    }
    return DG_OK;
}

int check_common(int n, int k, const void* b, const float* sb, const void* d) {
    if (n < 0 || k < 0) return DG_ERR_INVALID_ARG;
    if (k == 0 || k % kKBlock != 0) return DG_ERR_UNSUPPORTED;
    if (n % 16 != 0) return DG_ERR_UNSUPPORTED;
    if (n > 0 && (!b || !sb || !d)) return DG_ERR_INVALID_ARG;
    if ((b && !aligned16(b)) || (sb && !aligned16(sb)) || (d && !aligned16(d))) return DG_ERR_MISALIGNED;
    return DG_OK;
}

}  // namespace

extern "C" {

const char* dg_status_string(int status) {
    switch (status) {
        case DG_OK: return "DG_OK";
        case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG";
        case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
        case DG_ERR_MISALIGNED: return "DG_ERR_MISALIGNED";
        case DG_ERR_HIP: return "DG_ERR_HIP";
        default: return "DG_ERR_UNKNOWN";
    }
}

int dg_get_m_alignment(void) { return kMAlign; }

int dg_set_num_cus(int n) {
    if (n < 0) return DG_ERR_INVALID_ARG;
    g_cu_cap.store(n);
    return DG_OK;
}

int dg_get_num_cus(void) {
    int st = DG_OK;
    const DeviceInfo* dev = device_info(&st);
    if (!dev) {
        const int cap = g_cu_cap.load();
        return cap > 0 ? cap : st;
    }
    return effective_cus(dev->cus);
}

int dg_set_kernel_config(int config_id) {
    if (config_id == -1) {
        for (auto& f : g_forced_cfg) f = -1;
        return DG_OK;
    }
    int count = 0;
    const KernelConfig* cfgs = dg::kernel_configs(&count);
    for (int i = 0; i < count; ++i) {
        if (cfgs[i].id == config_id) {
            g_forced_cfg[cfgs[i].layout] = i;
            return DG_OK;
        }
    }
    return DG_ERR_INVALID_ARG;
}

static int check_quant(const void* x, int x_dtype, long ldx, int rows, int k, const void* q, long ldq,
                       const float* s) {
    if (rows < 0 || k < 0 || (x_dtype != DG_DTYPE_F32 && x_dtype != DG_DTYPE_BF16)) return DG_ERR_INVALID_ARG;
    if (k == 0 || k % kKBlock != 0) return DG_ERR_UNSUPPORTED;
    if (rows == 0) return DG_OK;
    if (!x || !q || !s) return DG_ERR_INVALID_ARG;
    if (ldx < k || ldq < k) return DG_ERR_INVALID_ARG;
    const long esz = x_dtype == DG_DTYPE_F32 ? 4 : 2;
    // the kernels address row r at r * ld elements: keep every such offset in 63 bits
    if (ldx > LONG_MAX / 4 / rows || ldq > LONG_MAX / 4 / rows) return DG_ERR_UNSUPPORTED;
    if (!aligned16(x) || ldx % (16 / esz) || (reinterpret_cast<uintptr_t>(q) & 7u) || ldq % 8 ||
        (reinterpret_cast<uintptr_t>(s) & 3u))
        return DG_ERR_MISALIGNED;
    return DG_OK;
}

int dg_quantize_fp8_1x128_fmt(const void* x, int x_dtype, long ldx, int rows, int k, void* q, long ldq, float* sa,
                              long ld_sa, int q_fmt, void* stream) {
    if (!valid_fmt(q_fmt)) return DG_ERR_INVALID_ARG;
    const int st = check_quant(x, x_dtype, ldx, rows, k, q, ldq, sa);
    if (st != DG_OK || rows == 0) return st;
    if (ld_sa < rows) return DG_ERR_INVALID_ARG;
    // sA exactly as the GEMMs take it: 16-byte aligned rows of the MN-major layout
    if (ld_sa % 4 || !aligned16(sa)) return DG_ERR_MISALIGNED;
    if (dg::launch_quant_1x128(x, x_dtype == DG_DTYPE_BF16, ldx, rows, k, static_cast<uint8_t*>(q), ldq, sa, ld_sa,
                               q_fmt == DG_FMT_E5M2, static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return DG_ERR_HIP;
    }
    return DG_OK;
}

int dg_quantize_fp8_1x128(const void* x, int x_dtype, long ldx, int rows, int k, void* q, long ldq, float* sa,
                          long ld_sa, void* stream) {
    return dg_quantize_fp8_1x128_fmt(x, x_dtype, ldx, rows, k, q, ldq, sa, ld_sa, DG_FMT_E4M3, stream);
}

int dg_quantize_fp8_128x128_fmt(const void* x, int x_dtype, long ldx, int rows, int k, void* q, long ldq, float* sb,
                                int q_fmt, void* stream) {
    if (!valid_fmt(q_fmt)) return DG_ERR_INVALID_ARG;
    const int st = check_quant(x, x_dtype, ldx, rows, k, q, ldq, sb);
    if (st != DG_OK || rows == 0) return st;
    if (dg::launch_quant_128x128(x, x_dtype == DG_DTYPE_BF16, ldx, rows, k, static_cast<uint8_t*>(q), ldq, sb,
                                 q_fmt == DG_FMT_E5M2, static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return DG_ERR_HIP;
    }
    return DG_OK;
}

int dg_quantize_fp8_128x128(const void* x, int x_dtype, long ldx, int rows, int k, void* q, long ldq, float* sb,
                            void* stream) {
    return dg_quantize_fp8_128x128_fmt(x, x_dtype, ldx, rows, k, q, ldq, sb, DG_FMT_E4M3, stream);
}

long dg_get_aligned_ld_sa(long rows) {
    if (rows < 0) return DG_ERR_INVALID_ARG;
    if (rows > LONG_MAX - 3) return DG_ERR_UNSUPPORTED;
    return (rows + 3) / 4 * 4;
}

int dg_transform_sa_mn_major(const float* sa_in, long ld_in, float* sa_out, long ld_sa, int rows, int kblocks,
                             int groups, void* stream) {
    if (rows < 0 || kblocks < 0 || groups < 1) return DG_ERR_INVALID_ARG;
    if (rows == 0 || kblocks == 0) return DG_OK;
    if (!sa_in || !sa_out || ld_in < kblocks || ld_sa < rows) return DG_ERR_INVALID_ARG;
    if (ld_sa % 4 || !aligned16(sa_out) || (reinterpret_cast<uintptr_t>(sa_in) & 3u)) return DG_ERR_MISALIGNED;
    if (ld_in > INT_MAX || ld_sa > INT_MAX || (long)rows * ld_in > INT_MAX || (long)kblocks * ld_sa > INT_MAX ||
        groups > 65535 || kblocks > 65535 * 32)
        return DG_ERR_UNSUPPORTED;
    if (dg::launch_sa_mn_major(sa_in, ld_in, sa_out, ld_sa, rows, kblocks, groups,
                               static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return DG_ERR_HIP;
    }
    return DG_OK;
}

int dg_check_contiguous_layout(const int* m_indices, int m_total, int num_groups, int* bad_row) {
    if (bad_row) *bad_row = -1;
    if (m_total < 0 || num_groups < 1 || (m_total > 0 && !m_indices)) return DG_ERR_INVALID_ARG;
    if (m_total % kMAlign != 0) {
        if (bad_row) *bad_row = m_total;
        return DG_ERR_INVALID_ARG;
    }
    for (int b = 0; b < m_total; b += kMAlign) {
        const int g = m_indices[b];
        for (int r = b; r < b + kMAlign; ++r) {
            const int v = m_indices[r];
            // entries are a group or -1; a block's group is that of its first row, and
            // every other row of the block is that group or padding
            const bool ok = v >= -1 && v < num_groups && (v == -1 || v == g);
            if (!ok) {
                if (bad_row) *bad_row = r;
                return DG_ERR_INVALID_ARG;
            }
        }
    }
    return DG_OK;
}

int dg_kernel_config_info(int index, int* out) {
    int count = 0;
    const KernelConfig* cfgs = dg::kernel_configs(&count);
    if (!out || index < 0 || index >= count) return DG_ERR_INVALID_ARG;
    out[0] = cfgs[index].id;
    out[1] = cfgs[index].layout;
    out[2] = cfgs[index].bm;
    out[3] = cfgs[index].bn;
    out[4] = cfgs[index].wm * cfgs[index].wn * cfgs[index].wk;
    out[5] = cfgs[index].all_formats ? 1 : 0;
    out[6] = cfgs[index].shape_specialised ? 1 : 0;
    out[7] = cfgs[index].wk;
    return DG_OK;
}

int dg_plan_tiles(int m, int n, int num_units, int blocks_per_unit, const int* block_ms, int n_bm,
                  const int* block_ns, int n_bn, const double* eff, int* out) {
    if (m <= 0 || n <= 0 || num_units <= 0 || blocks_per_unit <= 0 || !block_ms || !block_ns || n_bm <= 0 ||
        n_bn <= 0 || !out)
        return DG_ERR_INVALID_ARG;
    int best = -1;
    double best_cost = 0.0;
    long best_waves = 0;
    for (int i = 0; i < n_bm; ++i) {
        for (int j = 0; j < n_bn; ++j) {
            const int bm = block_ms[i], bn = block_ns[j];
            if (bm <= 0 || bn <= 0) return DG_ERR_INVALID_ARG;
            const double e = eff ? eff[i * n_bn + j] : 1.0;
            if (!(e > 0.0)) continue;
            const long tiles = ceil_div(m, bm) * ceil_div(n, bn);
            const long waves = ceil_div(tiles, (long)num_units * blocks_per_unit);
            const double cost = (double)waves * bm * bn / e;
            if (best < 0 || better(cost, waves, best_cost, best_waves)) {
                best = i * n_bn + j;
                best_cost = cost;
                best_waves = waves;
                out[0] = bm;
                out[1] = bn;
                out[2] = (int)tiles;
                out[3] = (int)waves;
            }
        }
    }
    return best < 0 ? DG_ERR_INVALID_ARG : best;
}

int dg_describe_launch(int layout, int m, int n, int k, int num_groups, int num_cus, int* out) {
    if (!out || m < 0 || n <= 0 || k <= 0 || num_groups < 1 || layout < 0 || layout > 2) return DG_ERR_INVALID_ARG;
    GemmParams p{};
    p.rows = m;
    p.n = n;
    p.k = k;
    p.kblocks = k / kKBlock;
    p.nblocks = (int)ceil_div(n, kKBlock);
    p.num_groups = layout == dg::kDense ? 1 : num_groups;
    const int units = num_cus > 0 ? effective_cus(num_cus) : 0;
    return launch(layout, p, m, m, nullptr, units, out);
}

int dg_gemm_fp8_nt_fmt(const void* a, long lda, const float* sa, long ld_sa, const void* b, long ldb, const float* sb,
                       void* d, long ldd, int m, int n, int k, int a_fmt, int b_fmt, void* stream) {
    if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
    int st = check_common(n, k, b, sb, d);
    if (st != DG_OK) return st;
    if (m < 0) return DG_ERR_INVALID_ARG;
    if (m == 0 || n == 0) return DG_OK;
    if (!a || !sa) return DG_ERR_INVALID_ARG;
    if (lda < k || ldb < k || ldd < n || ld_sa < m) return DG_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(sa) || lda % 16 || ldb % 16 || ldd % 8 || ld_sa % 4) return DG_ERR_MISALIGNED;
    if (!offsets_fit(lda, ldb, ld_sa, k) || (long)m * lda > LONG_MAX / 2 || ldd > LONG_MAX / 4 / m)
        return DG_ERR_UNSUPPORTED;
    GemmParams p{};
    p.a = static_cast<const uint8_t*>(a);
    p.lda = lda;
    p.sa = sa;
    p.ld_sa = ld_sa;
    p.b = static_cast<const uint8_t*>(b);
    p.ldb = ldb;
    p.sb = sb;
    p.d = static_cast<uint16_t*>(d);
    p.ldd = ldd;
    p.rows = m;
    p.n = n;
    p.k = k;
    p.kblocks = k / kKBlock;
    p.nblocks = (int)ceil_div(n, kKBlock);
    p.num_groups = 1;
    p.fmt = fmt_bits(a_fmt, b_fmt);
    return launch(dg::kDense, p, m, m, static_cast<hipStream_t>(stream), 0, nullptr);
}

int dg_gemm_fp8_nt(const void* a, long lda, const float* sa, long ld_sa, const void* b, long ldb, const float* sb,
                   void* d, long ldd, int m, int n, int k, void* stream) {
    return dg_gemm_fp8_nt_fmt(a, lda, sa, ld_sa, b, ldb, sb, d, ldd, m, n, k, DG_FMT_E4M3, DG_FMT_E4M3, stream);
}

int dg_m_grouped_gemm_fp8_contiguous_fmt(const void* a, const float* sa, long ld_sa, const void* b, const float* sb,
                                         void* d, const int* m_indices, int m_total, int n, int k, int num_groups,
                                         int a_fmt, int b_fmt, void* stream) {
    if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
    int st = check_common(n, k, b, sb, d);
    if (st != DG_OK) return st;
    if (m_total < 0 || num_groups < 1) return DG_ERR_INVALID_ARG;
    if (m_total % kMAlign != 0) return DG_ERR_INVALID_ARG;
    if (m_total == 0 || n == 0) return DG_OK;
    if (!a || !sa || !m_indices) return DG_ERR_INVALID_ARG;
    if (ld_sa < m_total) return DG_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(sa) || k % 16 || ld_sa % 4 || (reinterpret_cast<uintptr_t>(m_indices) & 3u))
        return DG_ERR_MISALIGNED;
    if (!offsets_fit(k, k, ld_sa, k)) return DG_ERR_UNSUPPORTED;
    GemmParams p{};
    p.a = static_cast<const uint8_t*>(a);
    p.lda = k;
    p.sa = sa;
    p.ld_sa = ld_sa;
    p.b = static_cast<const uint8_t*>(b);
    p.ldb = k;
    p.b_gstride = (long)n * k;
    p.sb = sb;
    p.sb_gstride = ceil_div(n, kKBlock) * (k / kKBlock);
    p.d = static_cast<uint16_t*>(d);
    p.ldd = n;
    p.m_indices = m_indices;
    p.rows = m_total;
    p.n = n;
    p.k = k;
    p.kblocks = k / kKBlock;
    p.nblocks = (int)ceil_div(n, kKBlock);
    p.num_groups = num_groups;
    p.fmt = fmt_bits(a_fmt, b_fmt);
    return launch(dg::kContiguous, p, m_total, m_total, static_cast<hipStream_t>(stream), 0, nullptr);
}

int dg_m_grouped_gemm_fp8_contiguous(const void* a, const float* sa, long ld_sa, const void* b, const float* sb,
                                     void* d, const int* m_indices, int m_total, int n, int k, int num_groups,
                                     void* stream) {
    return dg_m_grouped_gemm_fp8_contiguous_fmt(a, sa, ld_sa, b, sb, d, m_indices, m_total, n, k, num_groups,
                                                DG_FMT_E4M3, DG_FMT_E4M3, stream);
}

int dg_m_grouped_gemm_fp8_masked_fmt(const void* a, const float* sa, long ld_sa, const void* b, const float* sb,
                                     void* d, const int* masked_m, int num_groups, int max_m, int n, int k,
                                     int a_fmt, int b_fmt, void* stream) {
    if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
    int st = check_common(n, k, b, sb, d);
    if (st != DG_OK) return st;
    if (max_m < 0 || num_groups < 1) return DG_ERR_INVALID_ARG;
    if (num_groups > kMaxMaskedGroups) return DG_ERR_UNSUPPORTED;
    if (max_m == 0 || n == 0) return DG_OK;
    if (!a || !sa || !masked_m) return DG_ERR_INVALID_ARG;
    if (ld_sa < max_m) return DG_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(sa) || k % 16 || ld_sa % 4 || (reinterpret_cast<uintptr_t>(masked_m) & 3u))
        return DG_ERR_MISALIGNED;
    if (!offsets_fit(k, k, ld_sa, k)) return DG_ERR_UNSUPPORTED;
    GemmParams p{};
    p.a = static_cast<const uint8_t*>(a);
    p.lda = k;
    p.a_gstride = (long)max_m * k;
    p.sa = sa;
    p.ld_sa = ld_sa;
    p.sa_gstride = (long)(k / kKBlock) * ld_sa;
    p.b = static_cast<const uint8_t*>(b);
    p.ldb = k;
    p.b_gstride = (long)n * k;
    p.sb = sb;
    p.sb_gstride = ceil_div(n, kKBlock) * (k / kKBlock);
    p.d = static_cast<uint16_t*>(d);
    p.ldd = n;
    p.d_gstride = (long)max_m * n;
    p.masked_m = masked_m;
    p.rows = max_m;
    p.n = n;
    p.k = k;
    p.kblocks = k / kKBlock;
    p.nblocks = (int)ceil_div(n, kKBlock);
    p.num_groups = num_groups;
    p.fmt = fmt_bits(a_fmt, b_fmt);
    return launch(dg::kMasked, p, max_m, max_m, static_cast<hipStream_t>(stream), 0, nullptr);
}

int dg_m_grouped_gemm_fp8_masked(const void* a, const float* sa, long ld_sa, const void* b, const float* sb,
                                 void* d, const int* masked_m, int num_groups, int max_m, int n, int k,
                                 void* stream) {
    return dg_m_grouped_gemm_fp8_masked_fmt(a, sa, ld_sa, b, sb, d, masked_m, num_groups, max_m, n, k,
                                            DG_FMT_E4M3, DG_FMT_E4M3, stream);
}

}  // extern "C"
