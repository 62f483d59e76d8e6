"""Host-side checks of libdg.so that need no GPU: it loads, exports every symbol
the public header declares, validates arguments before touching a device, and its
tile planner reproduces the pages' unaligned-block-size example."""
import ctypes
import os
import re

import pytest

import fp8_block_scaled_e4m3_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("dg.h", "dg_tuning.h")]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lib():
    return dg.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
        assert hasattr(dg, name), f"python binding lacks {name}"


def test_status_strings(lib):
    assert dg.status_string(0) == "DG_OK"
    for code, name in [(-1, "DG_ERR_INVALID_ARG"), (-2, "DG_ERR_UNSUPPORTED"), (-3, "DG_ERR_MISALIGNED"),
                       (-4, "DG_ERR_HIP")]:
        assert dg.status_string(code) == name
    assert dg.status_string(12345) == "DG_ERR_UNKNOWN"


def test_m_alignment_and_cu_cap(lib):
    assert dg.dg_get_m_alignment() == 128
    assert lib.dg_set_num_cus(-1) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_set_num_cus(100) == 0
    assert lib.dg_get_num_cus() == 100            # no device here: the cap is reported
    assert lib.dg_set_num_cus(0) == 0


def test_kernel_configs_listed(lib):
    cfgs = dg.dg_kernel_config_info()
    layouts = {c["layout"] for c in cfgs}
    assert layouts == {0, 1, 2}
    for c in cfgs:
        assert c["block_m"] % 16 == 0 and c["block_n"] % 16 == 0
        if c["layout"] == 1:
            # a tile lies inside one 128-row segment block or covers exactly two
            # (computed in one pass per group when they differ)
            assert 128 % c["block_m"] == 0 or c["block_m"] == 256
    assert lib.dg_set_kernel_config(999) == dg.DG_ERR_INVALID_ARG
    assert lib.dg_set_kernel_config(-1) == 0


def _call_dense(lib, a=16, sa=16, b=16, sb=16, d=16, lda=512, ld_sa=128, ldb=512, ldd=128, m=128, n=128, k=512):
    P = ctypes.c_void_p
    return lib.dg_gemm_fp8_nt(P(a), lda, P(sa), ld_sa, P(b), ldb, P(sb), P(d), ldd, m, n, k, None)


def _call_dense_fmt(lib, a_fmt, b_fmt, k=512):
    P = ctypes.c_void_p
    return lib.dg_gemm_fp8_nt_fmt(P(16), 512, P(16), 128, P(16), 512, P(16), P(16), 128, 128, 128, k,
                                  a_fmt, b_fmt, None)


def _call_grouped_fmt(lib, layout, a_fmt, b_fmt, k=512):
    P = ctypes.c_void_p
    if layout == 1:
        return lib.dg_m_grouped_gemm_fp8_contiguous_fmt(P(16), P(16), 128, P(16), P(16), P(16), P(16),
                                                        128, 128, k, 2, a_fmt, b_fmt, None)
    return lib.dg_m_grouped_gemm_fp8_masked_fmt(P(16), P(16), 128, P(16), P(16), P(16), P(16),
                                                2, 128, 128, k, a_fmt, b_fmt, None)


def test_format_entry_validation(lib):
    """Unknown format codes are rejected before anything else, in every layout; every
    layout has configurations that carry the E5M2 variants."""
    assert (dg.DG_FMT_E4M3, dg.DG_FMT_E5M2) == (0, 1)
    for fa, fb in ((2, 0), (0, -1), (7, 7)):
        assert _call_dense_fmt(lib, fa, fb) == dg.DG_ERR_INVALID_ARG
        assert _call_grouped_fmt(lib, 1, fa, fb) == dg.DG_ERR_INVALID_ARG
        assert _call_grouped_fmt(lib, 2, fa, fb) == dg.DG_ERR_INVALID_ARG
    for fa, fb in ((0, 1), (1, 0), (1, 1)):
        assert _call_dense_fmt(lib, fa, fb, k=500) == dg.DG_ERR_UNSUPPORTED
        assert _call_grouped_fmt(lib, 1, fa, fb, k=500) == dg.DG_ERR_UNSUPPORTED
        assert _call_grouped_fmt(lib, 2, fa, fb, k=500) == dg.DG_ERR_UNSUPPORTED
    cfgs = dg.dg_kernel_config_info()
    for layout in (0, 1, 2):
        assert any(c["all_formats"] for c in cfgs if c["layout"] == layout)
        assert not all(c["all_formats"] for c in cfgs if c["layout"] == layout)


def test_dense_validation_before_any_device_work(lib):
    assert _call_dense(lib, k=500) == dg.DG_ERR_UNSUPPORTED
    assert _call_dense(lib, k=0) == dg.DG_ERR_UNSUPPORTED
    assert _call_dense(lib, n=120, ldd=128) == dg.DG_ERR_UNSUPPORTED
    assert _call_dense(lib, m=-1) == dg.DG_ERR_INVALID_ARG
    assert _call_dense(lib, a=0) == dg.DG_ERR_INVALID_ARG
    assert _call_dense(lib, b=0) == dg.DG_ERR_INVALID_ARG
    assert _call_dense(lib, a=24) == dg.DG_ERR_MISALIGNED
    assert _call_dense(lib, lda=520) == dg.DG_ERR_MISALIGNED
    assert _call_dense(lib, ldd=130) == dg.DG_ERR_MISALIGNED
    assert _call_dense(lib, ld_sa=64) == dg.DG_ERR_INVALID_ARG
    assert _call_dense(lib, lda=256) == dg.DG_ERR_INVALID_ARG
    assert _call_dense(lib, m=0) == dg.DG_OK           # empty problem: no-op, no device needed


def test_size_limits_of_32bit_offsets(lib):
    """Sizes whose per-tile offsets would not fit in 32 bits are refused on the host
    (before any device work), in every layout."""
    P = ctypes.c_void_p
    k = 7168
    big_ld = (0xFFFFFFFF - k) // 256 + 16          # 256 * ld + k just past 2^32
    assert _call_dense(lib, lda=big_ld - big_ld % 16, ldb=k, k=k, ld_sa=128) == dg.DG_ERR_UNSUPPORTED
    assert _call_dense(lib, lda=k, ldb=big_ld - big_ld % 16, k=k, ld_sa=128) == dg.DG_ERR_UNSUPPORTED
    # A scales: (k/128) * ld_sa * 4 past 2^32 (rows that would fit in HBM at small N)
    rows = (0xFFFFFFFF // (4 * (k // 128))) // 4 * 4 + 4
    assert _call_dense(lib, m=rows, lda=k, ldb=k, ld_sa=rows, k=k) == dg.DG_ERR_UNSUPPORTED
    assert lib.dg_m_grouped_gemm_fp8_contiguous(P(16), P(16), rows + 124, P(16), P(16), P(16), P(16),
                                                (rows // 128 + 1) * 128, 128, k, 2, None) == dg.DG_ERR_UNSUPPORTED
    assert lib.dg_m_grouped_gemm_fp8_masked(P(16), P(16), rows, P(16), P(16), P(16), P(16),
                                            2, rows, 128, k, None) == dg.DG_ERR_UNSUPPORTED


def test_grouped_validation(lib):
    P = ctypes.c_void_p
    c = lib.dg_m_grouped_gemm_fp8_contiguous
    assert c(P(16), P(16), 256, P(16), P(16), P(16), P(16), 200, 128, 256, 2, None) == dg.DG_ERR_INVALID_ARG
    assert c(P(16), P(16), 256, P(16), P(16), P(16), P(16), 256, 128, 256, 0, None) == dg.DG_ERR_INVALID_ARG
    assert c(P(16), P(16), 256, P(16), P(16), P(16), None, 256, 128, 256, 2, None) == dg.DG_ERR_INVALID_ARG
    assert c(P(16), P(16), 256, P(16), P(16), P(16), P(16), 0, 128, 256, 2, None) == dg.DG_OK
    mk = lib.dg_m_grouped_gemm_fp8_masked
    assert mk(P(16), P(16), 256, P(16), P(16), P(16), P(16), 2, 256, 128, 100, None) == dg.DG_ERR_UNSUPPORTED
    assert mk(P(16), P(16), 256, P(16), P(16), P(16), P(16), 2000, 256, 128, 256, None) == dg.DG_ERR_UNSUPPORTED
    assert mk(P(16), P(16), 100, P(16), P(16), P(16), P(16), 2, 256, 128, 256, None) == dg.DG_ERR_INVALID_ARG
    assert mk(P(16), P(16), 256, P(16), P(16), P(16), P(16), 2, 0, 128, 256, None) == dg.DG_OK


def test_plan_reproduces_unaligned_block_example(lib):
    """The pages' worked example: M=256, N=7168, BLOCK_M=128 on 132 units -- 128x128 tiles
    fill 112 units, 128x112 tiles fill 128, and the planner prefers the latter."""
    rows = []
    for line in open(os.path.join(GOLDEN, "unaligned_block_fill.txt")):
        if line.strip() and not line.startswith("#"):
            rows.append([int(x) for x in line.split()])
    for m, n, units, bm, bn, tiles in rows:
        _, pbm, pbn, ptiles, waves = dg.dg_plan_tiles(m, n, units, [bm], [bn])
        assert (pbm, pbn, ptiles, waves) == (bm, bn, tiles, 1)
    m, n, units = rows[0][:3]
    _, bm, bn, tiles, waves = dg.dg_plan_tiles(m, n, units, [128], list(range(16, 257, 16)))
    assert (bm, bn, tiles, waves) == (128, 112, 128, 1)


def test_plan_fills_256_cus():
    _, bm, bn, tiles, waves = dg.dg_plan_tiles(256, 7168, 256, [64, 128], list(range(16, 257, 16)))
    assert (bm, bn, tiles, waves) == (64, 112, 256, 1)


def test_describe_launch_shapes():
    # 256x256 tiles (one B scale row per wave) beat 256x224 (two whole rounds) in the
    # planner's model: 448 tiles, the second round three quarters full
    d = dg.dg_describe_launch(0, 4096, 7168, 7168, 1, 256)
    assert (d["block_m"], d["block_n"], d["tiles"]) == (256, 256, 448) and d["grid"] == 256
    # each XCD takes 32 consecutive tiles per round: 8 row tiles x 4 column tiles, and
    # 8 x 28 = 224 tiles per raster group is a multiple of 32 (4 would straddle groups)
    assert d["group_m"] == 8
    d = dg.dg_describe_launch(0, 256, 7168, 2048, 1, 256)
    assert (d["block_m"], d["block_n"], d["tiles"]) == (64, 112, 256)
    assert d["group_m"] == 4                    # 4 row tiles x 8 column tiles of 64x112
    d = dg.dg_describe_launch(1, 33280, 4096, 7168, 8, 256)
    assert (d["block_m"], d["block_n"], d["tiles"]) == (256, 256, 130 * 16)
    d = dg.dg_describe_launch(2, 256, 4096, 7168, 16, 256)
    assert d["block_m"] == 256 and d["tiles"] == 16 * 4096 // d["block_n"]
    # a CU cap below the 256 tiles of 256x256 picks the narrower tiles (fewer rounds)
    assert (d["block_n"], d["grid"]) == (256, 256)
    d = dg.dg_describe_launch(2, 256, 4096, 7168, 16, 224)
    assert (d["block_m"], d["block_n"], d["grid"]) == (256, 128, 224)


def test_describe_launch_k_groups():
    """Two wave groups over alternate K blocks (k_groups 2) only where the tiles leave
    CUs idle or just fill them and K is long: 64x4096x7168 (64 tiles of 64x64) and
    128x7168x7168 (224) take them; the same shapes at K = 2048, or with more tiles than
    CUs, keep one chain."""
    groups = {c["id"]: c["k_groups"] for c in dg.dg_kernel_config_info()}
    assert sorted(set(groups.values())) == [1, 2]
    assert all(c["layout"] == 0 for c in dg.dg_kernel_config_info() if c["k_groups"] == 2)
    for m, n, k, want in ((64, 4096, 7168, 2), (128, 7168, 7168, 2), (64, 4096, 4096, 2), (64, 4096, 2048, 1),
                          (256, 7168, 2048, 1), (512, 4096, 7168, 1), (4096, 7168, 7168, 1)):
        d = dg.dg_describe_launch(0, m, n, k, 1, 256)
        assert groups[d["config_id"]] == want, (m, n, k, d)
        if want == 2:
            assert d["tiles"] <= 256 and d["waves_per_workgroup"] == 8
    # a CU cap below the tile count drops them
    d = dg.dg_describe_launch(0, 128, 7168, 7168, 1, 200)
    assert groups[d["config_id"]] == 1


def test_describe_reports_shape_instances():
    """The V3 shapes run instances compiled for their N and K: dense N = 7168 with
    K = 7168 or 2048, contiguous and masked N = 4096 with K = 7168; another N or K, and
    configurations without such instances, run the generic kernel."""
    info = dg.dg_kernel_config_info()
    specs = {c["id"] for c in info if c["shape_specialised"]}
    assert {c["layout"] for c in info if c["shape_specialised"]} == {0, 1, 2}
    d = dg.dg_describe_launch(0, 4096, 7168, 7168, 1, 256)
    assert d["config_id"] in specs and d["k_blocks_specialised"] == 56
    d = dg.dg_describe_launch(0, 256, 7168, 2048, 1, 256)
    assert d["config_id"] in specs and d["k_blocks_specialised"] == 16
    d = dg.dg_describe_launch(1, 33280, 4096, 7168, 8, 256)
    assert d["config_id"] in specs and d["k_blocks_specialised"] == 56
    d = dg.dg_describe_launch(2, 256, 4096, 7168, 16, 256)
    assert d["config_id"] in specs and d["k_blocks_specialised"] == 56
    assert dg.dg_describe_launch(0, 4096, 7168, 4096, 1, 256)["k_blocks_specialised"] == 0
    assert dg.dg_describe_launch(0, 4096, 4096, 7168, 1, 256)["k_blocks_specialised"] == 0
    assert dg.dg_describe_launch(1, 33280, 7168, 2048, 8, 256)["k_blocks_specialised"] == 0
    assert dg.dg_describe_launch(2, 256, 4096, 2048, 16, 256)["k_blocks_specialised"] == 0


def test_quantize_validation(lib):
    P = ctypes.c_void_p
    q1 = lib.dg_quantize_fp8_1x128
    assert q1(P(16), 0, 256, 4, 200, P(16), 256, P(16), 4, None) == dg.DG_ERR_UNSUPPORTED
    assert q1(P(16), 7, 256, 4, 256, P(16), 256, P(16), 4, None) == dg.DG_ERR_INVALID_ARG
    assert q1(P(16), 0, 256, 4, 256, P(16), 256, P(16), 2, None) == dg.DG_ERR_INVALID_ARG     # ld_sa < rows
    assert q1(P(16), 0, 256, 4, 256, P(20), 256, P(16), 4, None) == dg.DG_ERR_MISALIGNED      # q not 8-aligned
    assert q1(P(16), 0, 257, 4, 256, P(16), 256, P(16), 4, None) == dg.DG_ERR_MISALIGNED      # ldx*4 % 16
    assert q1(None, 0, 256, 4, 256, P(16), 256, P(16), 4, None) == dg.DG_ERR_INVALID_ARG
    assert q1(P(16), 0, 256, 0, 256, P(16), 256, P(16), 4, None) == dg.DG_OK                  # empty: no-op
    q2 = lib.dg_quantize_fp8_128x128
    assert q2(P(16), 1, 256, 4, 384, P(16), 384, P(16), None) == dg.DG_ERR_INVALID_ARG       # ldx < k
    assert q2(P(16), 1, 388, 4, 384, P(16), 384, P(16), None) == dg.DG_ERR_MISALIGNED        # ldx*2 % 16
    assert q2(P(16), 1, 384, 0, 384, P(16), 384, P(16), None) == dg.DG_OK
    # output format: unknown codes rejected first; the E5M2 forms validate like the plain ones
    q1f, q2f = lib.dg_quantize_fp8_1x128_fmt, lib.dg_quantize_fp8_128x128_fmt
    assert q1f(P(16), 0, 256, 4, 256, P(16), 256, P(16), 4, 2, None) == dg.DG_ERR_INVALID_ARG
    assert q2f(P(16), 0, 256, 4, 256, P(16), 256, P(16), -1, None) == dg.DG_ERR_INVALID_ARG
    assert q1f(P(16), 0, 256, 4, 200, P(16), 256, P(16), 4, 1, None) == dg.DG_ERR_UNSUPPORTED
    assert q2f(P(16), 1, 388, 4, 384, P(16), 384, P(16), 1, None) == dg.DG_ERR_MISALIGNED
    assert q1f(P(16), 0, 256, 0, 256, P(16), 256, P(16), 4, 1, None) == dg.DG_OK


def test_quantize_1x128_takes_only_an_sa_the_gemm_accepts(lib):
    P = ctypes.c_void_p
    q1 = lib.dg_quantize_fp8_1x128
    assert q1(P(16), 0, 256, 6, 256, P(16), 256, P(16), 6, None) == dg.DG_ERR_MISALIGNED      # ld_sa % 4
    assert q1(P(16), 0, 256, 6, 256, P(16), 256, P(20), 8, None) == dg.DG_ERR_MISALIGNED      # sa not 16-aligned
    assert q1(P(16), 0, 256, 6, 256, P(16), 256, P(16), 5, None) == dg.DG_ERR_INVALID_ARG     # ld_sa < rows
    assert lib.dg_quantize_fp8_1x128_fmt(P(16), 0, 256, 6, 256, P(16), 256, P(16), 6, 1, None) == \
        dg.DG_ERR_MISALIGNED


def test_aligned_ld_sa():
    assert [dg.dg_get_aligned_ld_sa(r) for r in (0, 1, 3, 4, 5, 4096, 4097)] == [0, 4, 4, 4, 8, 4096, 4100]
    with pytest.raises(dg.DGError):
        dg.dg_get_aligned_ld_sa(-1)


def test_transform_sa_validation(lib):
    P = ctypes.c_void_p
    t = lib.dg_transform_sa_mn_major
    assert t(P(16), 55, P(16), 4096, 4096, 56, 1, None) == dg.DG_ERR_INVALID_ARG   # ld_in < kblocks
    assert t(P(16), 56, P(16), 4095, 4096, 56, 1, None) == dg.DG_ERR_INVALID_ARG   # ld_sa < rows
    assert t(P(16), 56, P(16), 4098, 4097, 56, 1, None) == dg.DG_ERR_MISALIGNED    # ld_sa % 4
    assert t(P(16), 56, P(24), 4100, 4097, 56, 1, None) == dg.DG_ERR_MISALIGNED    # out not 16-aligned
    assert t(P(18), 56, P(16), 4100, 4097, 56, 1, None) == dg.DG_ERR_MISALIGNED    # in not 4-aligned
    assert t(None, 56, P(16), 4100, 4097, 56, 1, None) == dg.DG_ERR_INVALID_ARG
    assert t(P(16), 56, P(16), 4100, 4097, 56, 0, None) == dg.DG_ERR_INVALID_ARG   # groups < 1
    assert t(P(16), 56, P(16), 4100, 4097, 56, 70000, None) == dg.DG_ERR_UNSUPPORTED
    assert t(P(16), 56, P(16), 4100, 0, 56, 1, None) == dg.DG_OK                   # empty: no-op
    assert t(P(16), 56, P(16), 4100, 4097, 0, 1, None) == dg.DG_OK


def test_contiguous_layout_checker():
    import numpy as np

    def layout(counts, ng):
        mi = []
        for g, c in enumerate(counts):
            p = -(-c // 128) * 128
            mi += [g] * c + [-1] * (p - c)
        return np.array(mi, np.int32), ng

    mi, ng = layout([130, 0, 1, 257, 128], 5)
    assert dg.dg_check_contiguous_layout(mi, ng) is None
    assert dg.dg_check_contiguous_layout(np.zeros(0, np.int32), 1) is None
    assert dg.dg_check_contiguous_layout(mi[:200], ng) == 200            # not a multiple of 128
    bad = mi.copy(); bad[5] = 7                                           # group out of range
    assert dg.dg_check_contiguous_layout(bad, ng) == 5
    bad = mi.copy(); bad[3] = -2                                          # not a group, not -1
    assert dg.dg_check_contiguous_layout(bad, ng) == 3
    bad = mi.copy(); bad[129] = 3                                         # another group inside a block
    assert dg.dg_check_contiguous_layout(bad, ng) == 129
    bad = mi.copy(); bad[384] = -1                                        # block starts with padding ...
    assert dg.dg_check_contiguous_layout(bad, ng) == 385                  # ... but holds rows of group 3
    ok = mi.copy(); ok[130:140] = 0; ok[135] = -1                         # padding between rows of the group
    assert dg.dg_check_contiguous_layout(ok, ng) is None


def test_readme_python_names_host_side():
    """The README's utility names: the TMA-aligned size is the aligned ld_sa for fp32
    scales (16 bytes), generic in the element size; the contiguous alignment is 128."""
    for x in (1, 3, 4, 5, 301, 4096, 4097):
        assert dg.get_tma_aligned_size(x, 4) == dg.dg_get_aligned_ld_sa(x)
    assert dg.get_tma_aligned_size(10, 2) == 16 and dg.get_tma_aligned_size(16, 1) == 16
    with pytest.raises(ValueError):
        dg.get_tma_aligned_size(10, 3)
    assert dg.get_m_alignment_for_contiguous_layout() == dg.dg_get_m_alignment() == 128
