"""GPU parity for the GEMMs with E5M2 operands (either side, or both).

The blog's FP8 section lets each operand be E4M3 or E5M2.  Every combination is
compared with the oracle element by element on small and ragged shapes in each
tile configuration that carries the E5M2 variants (dense, contiguous and masked
layouts), through the planner, and on a larger dense shape on sampled rows; the
E4M3/E4M3 case of each _fmt entry point must be bit-identical to the plain one.
"""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, sample_rows, say, sentinel_like, upload

pytestmark = pytest.mark.gpu

COMBOS = [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    dev = require_gpu()
    dg.load_library()
    yield dev
    dg.dg_set_kernel_config(-1)
    dg.dg_set_num_cus(0)


def fmt_configs(layout=0):
    return [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == layout and c["all_formats"]]


def run_fmt(dd, cfg=-1, pad_cols=16):
    import torch
    dv = upload(dd)
    m, n = dd["a"].shape[0], dd["b"].shape[0]
    full = sentinel_like((m, n + pad_cols))
    dg.dg_set_kernel_config(cfg)
    try:
        dg.dg_gemm_fp8_nt_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], full[:, :n],
                              a_fmt=dd["a_fmt"], b_fmt=dd["b_fmt"])
        torch.cuda.synchronize()
    finally:
        dg.dg_set_kernel_config(-1)
    fb = bits(full)
    return fb[:, :n], fb


def oracle_fmt(orc, dd, rows=None):
    a, sa = dd["a"], dd["sa"]
    if rows is not None:
        a, sa = a[rows], sa[:, rows]
    return orc.gemm_fp8_nt(a, sa, dd["b"], dd["sb"], a_fmt=dd["a_fmt"], b_fmt=dd["b_fmt"])


def test_format_configs_exist():
    assert len(fmt_configs(0)) >= 2 and len(fmt_configs(1)) >= 2 and len(fmt_configs(2)) >= 2


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (128, 128, 512), (300, 208, 384), (513, 1040, 1024)])
def test_e5m2_ragged_shapes(orc, a_fmt, b_fmt, m, n, k):
    dd = W.make_dense(m, n, k, seed=7 * m + n + k, a_fmt=a_fmt, b_fmt=b_fmt)
    ref = oracle_fmt(orc, dd)
    groups = {c["id"]: c["k_groups"] for c in dg.dg_kernel_config_info()}
    first = {}
    for cfg in [-1] + fmt_configs():
        say(f"dense {a_fmt}x{b_fmt} {m}x{n}x{k} cfg={cfg}")
        out, full = run_fmt(dd, cfg)
        check_values(out, ref, f"{a_fmt}x{b_fmt} {m}x{n}x{k} cfg{cfg}")
        assert np.all(full[:, n:] == W.SENTINEL_BF16), "wrote past column n"
        # identical bits within a summation class (one chain, or two K groups added at the end)
        cls = groups[dg.dg_describe_launch(0, m, n, k, 1)["config_id"] if cfg == -1 else cfg]
        if cls in first:
            assert np.array_equal(out, first[cls])
        else:
            first[cls] = out


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
def test_e5m2_k_groups_planned(orc, a_fmt, b_fmt):
    """An under-filled long-K shape plans the two-K-group configuration for E5M2 operands
    as for E4M3: the whole output against the oracle."""
    m, n, k = 64, 2048, 4096
    d = dg.dg_describe_launch(0, m, n, k, 1)
    assert {c["id"]: c["k_groups"] for c in dg.dg_kernel_config_info()}[d["config_id"]] == 2, d
    dd = W.make_dense(m, n, k, seed=41, a_fmt=a_fmt, b_fmt=b_fmt)
    say(f"dense {a_fmt}x{b_fmt} {m}x{n}x{k} planned cfg={d['config_id']}")
    out, full = run_fmt(dd)
    assert np.all(full[:, n:] == W.SENTINEL_BF16)
    check_values(out, oracle_fmt(orc, dd), f"{a_fmt}x{b_fmt} {m}x{n}x{k} k groups")


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
def test_e5m2_chained_tiles(orc, a_fmt, b_fmt):
    """Few workgroups, many tiles each, K/128 a multiple of the stage count so the
    prefetch of the next tile runs across tile boundaries."""
    dd = W.make_dense(300, 464, 512, seed=91, a_fmt=a_fmt, b_fmt=b_fmt)
    ref = oracle_fmt(orc, dd)
    dg.dg_set_num_cus(3)
    try:
        for cfg in fmt_configs():
            say(f"dense {a_fmt}x{b_fmt} 300x464x512 cfg={cfg} cu cap 3")
            out, _ = run_fmt(dd, cfg)
            check_values(out, ref, f"{a_fmt}x{b_fmt} chained cfg{cfg}")
    finally:
        dg.dg_set_num_cus(0)


def test_e5m2_large_sampled(orc):
    dd = W.make_dense(2048, 4096, 2048, seed=5, a_fmt="e5m2", b_fmt="e4m3")
    say("dense e5m2xe4m3 2048x4096x2048 planned")
    out, full = run_fmt(dd)
    assert np.all(full[:, 4096:] == W.SENTINEL_BF16)
    rows = sample_rows(2048, 256, 32)
    check_values(out[rows], oracle_fmt(orc, dd, rows), "e5m2xe4m3 2048x4096x2048 sampled rows")


@pytest.mark.parametrize("k", [7168, 2048])
def test_e5m2_shape_instances(orc, k):
    """At N = 7168 with K = 7168 and K = 2048 the E5M2 calls run the instances compiled
    for that shape (pipelined where the K blocks split into stage groups): equal to the
    oracle, and equal across the configurations carrying them, with one tile per
    workgroup and with tiles chained on three workgroups."""
    dd = W.make_dense(300, 7168, k, seed=k + 17, a_fmt="e5m2", b_fmt="e4m3")
    ref = oracle_fmt(orc, dd)
    specs = [c["id"] for c in dg.dg_kernel_config_info()
             if c["layout"] == 0 and c["shape_specialised"] and c["all_formats"]]
    assert specs
    outs = []
    try:
        for cap in (0, 3):
            dg.dg_set_num_cus(cap)
            for cfg in specs:
                say(f"dense e5m2xe4m3 300x464x{k} cfg={cfg} cu cap {cap}")
                out, _ = run_fmt(dd, cfg)
                check_values(out, ref, f"e5m2 K={k} cfg{cfg} cap {cap}")
                outs.append(out)
    finally:
        dg.dg_set_num_cus(0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_e4m3_pair_matches_plain_entry():
    import torch
    dd = W.make_dense(200, 336, 640, seed=3)
    dv = upload(dd)
    d0 = torch.zeros((200, 336), dtype=torch.bfloat16, device="cuda:0")
    d1 = torch.ones((200, 336), dtype=torch.bfloat16, device="cuda:0")
    dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], d0)
    dg.dg_gemm_fp8_nt_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], d1, a_fmt="e4m3", b_fmt="e4m3")
    torch.cuda.synchronize()
    assert np.array_equal(bits(d0), bits(d1))


def test_float8_dtypes_carry_the_format(orc):
    import torch
    dd = W.make_dense(64, 128, 256, seed=11, a_fmt="e5m2", b_fmt="e5m2")
    dv = upload(dd)
    a8, b8 = dv["a"].view(torch.float8_e5m2), dv["b"].view(torch.float8_e5m2)
    d = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda:0")
    dg.dg_gemm_fp8_nt_fmt(a8, dv["sa"], b8, dv["sb"], d)
    torch.cuda.synchronize()
    check_values(bits(d), oracle_fmt(orc, dd), "float8_e5m2 tensors")
    with pytest.raises(ValueError):
        dg.dg_gemm_fp8_nt_fmt(a8, dv["sa"], b8, dv["sb"], d, a_fmt="e4m3")


def test_forced_config_without_formats_is_unsupported():
    import torch
    plain = [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 0 and not c["all_formats"]]
    assert plain
    dd = W.make_dense(64, 128, 256, seed=12, a_fmt="e5m2", b_fmt="e4m3")
    dv = upload(dd)
    d = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda:0")
    dg.dg_set_kernel_config(plain[0])
    try:
        with pytest.raises(dg.DGError) as e:
            dg.dg_gemm_fp8_nt_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], d, a_fmt="e5m2", b_fmt="e4m3")
    finally:
        dg.dg_set_kernel_config(-1)
    assert e.value.status == dg.DG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(d).item() == 0


# --------------------------------------------------------------------------- grouped layouts
def run_contiguous_fmt(cd, cfg=-1, a_fmt=None, b_fmt=None):
    import torch
    dv = upload(cd)
    out = sentinel_like((cd["m_total"], cd["n"]))
    dg.dg_set_kernel_config(cfg)
    try:
        dg.dg_m_grouped_gemm_fp8_contiguous_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["m_indices"],
                                                a_fmt=a_fmt or cd["a_fmt"], b_fmt=b_fmt or cd["b_fmt"])
        torch.cuda.synchronize()
    finally:
        dg.dg_set_kernel_config(-1)
    return bits(out)


def run_masked_fmt(md, cfg=-1, a_fmt=None, b_fmt=None):
    import torch
    dv = upload(md)
    out = sentinel_like((md["groups"], md["max_m"], md["n"]))
    dg.dg_set_kernel_config(cfg)
    try:
        dg.dg_m_grouped_gemm_fp8_masked_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"],
                                            a_fmt=a_fmt or md["a_fmt"], b_fmt=b_fmt or md["b_fmt"])
        torch.cuda.synchronize()
    finally:
        dg.dg_set_kernel_config(-1)
    return bits(out)


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
def test_e5m2_contiguous(orc, a_fmt, b_fmt):
    counts = [130, 0, 3, 257]
    cd = W.make_contiguous(counts, n=208, k=384, seed=31, a_fmt=a_fmt, b_fmt=b_fmt)
    sentinel = np.full((cd["m_total"], 208), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel,
                                   a_fmt=a_fmt, b_fmt=b_fmt)
    valid = cd["m_indices"] >= 0
    outs = []
    for cfg in [-1] + fmt_configs(1):
        say(f"contiguous {a_fmt}x{b_fmt} counts={counts} n=208 k=384 cfg={cfg}")
        out = run_contiguous_fmt(cd, cfg)
        check_values(out[valid], ref[valid], f"contiguous {a_fmt}x{b_fmt} cfg{cfg}")
        assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
def test_e5m2_masked(orc, a_fmt, b_fmt):
    mm = [0, 1, 70, 256, 129]
    md = W.make_masked(5, 256, 208, 384, seed=32, masked_m=mm, a_fmt=a_fmt, b_fmt=b_fmt)
    sentinel = np.full((5, 256, 208), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], md["masked_m"], d_init=sentinel,
                               a_fmt=a_fmt, b_fmt=b_fmt)
    outs = []
    for cfg in [-1] + fmt_configs(2):
        say(f"masked {a_fmt}x{b_fmt} masked_m={mm} n=208 k=384 cfg={cfg}")
        out = run_masked_fmt(md, cfg)
        for g, c in enumerate(mm):
            assert np.all(out[g, c:] == W.SENTINEL_BF16), f"group {g}: a row >= masked_m was written"
            if c:
                check_values(out[g, :c], ref[g, :c], f"masked {a_fmt}x{b_fmt} cfg{cfg} group {g}")
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("layout,a_fmt,b_fmt", [(1, "e5m2", "e4m3"), (2, "e4m3", "e5m2")])
def test_e5m2_grouped_shape_instances(orc, layout, a_fmt, b_fmt):
    """N = 4096 with K = 7168 runs the grouped configurations' shape instances with an
    E5M2 operand: equal to the oracle, and equal across every configuration of the layout
    that runs E5M2 (planned or pinned)."""
    info = {c["id"]: c for c in dg.dg_kernel_config_info()}
    assert any(info[c]["shape_specialised"] for c in fmt_configs(layout))
    outs = []
    if layout == 1:
        counts = [130, 0, 40]
        cd = W.make_contiguous(counts, n=4096, k=7168, seed=71, a_fmt=a_fmt, b_fmt=b_fmt)
        sentinel = np.full((cd["m_total"], 4096), W.SENTINEL_BF16, np.uint16)
        ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel,
                                       a_fmt=a_fmt, b_fmt=b_fmt)
        valid = cd["m_indices"] >= 0
        for cfg in [-1] + fmt_configs(1):
            say(f"contiguous {a_fmt}x{b_fmt} counts={counts} n=4096 k=7168 cfg={cfg}")
            out = run_contiguous_fmt(cd, cfg)
            assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
            outs.append(out)
        check_values(outs[0][valid], ref[valid], f"contiguous {a_fmt}x{b_fmt} n=4096 k=7168")
    else:
        mm = [0, 218, 77]
        md = W.make_masked(3, 256, 4096, 7168, seed=72, masked_m=mm, a_fmt=a_fmt, b_fmt=b_fmt)
        sentinel = np.full((3, 256, 4096), W.SENTINEL_BF16, np.uint16)
        ref = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], md["masked_m"], d_init=sentinel,
                                   a_fmt=a_fmt, b_fmt=b_fmt)
        for cfg in [-1] + fmt_configs(2):
            say(f"masked {a_fmt}x{b_fmt} masked_m={mm} n=4096 k=7168 cfg={cfg}")
            out = run_masked_fmt(md, cfg)
            for g, c in enumerate(mm):
                assert np.all(out[g, c:] == W.SENTINEL_BF16), f"group {g}: a row >= masked_m was written"
            outs.append(out)
        valid = np.arange(256)[None, :] < np.array(mm)[:, None]
        check_values(outs[0][valid], ref[valid], f"masked {a_fmt}x{b_fmt} n=4096 k=7168")
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_grouped_e4m3_pair_matches_plain_entries():
    import torch
    cd = W.make_contiguous([100, 40], n=96, k=256, seed=33)
    dv = upload(cd)
    o0, o1 = sentinel_like((cd["m_total"], 96)), sentinel_like((cd["m_total"], 96))
    dg.dg_m_grouped_gemm_fp8_contiguous(dv["a"], dv["sa"], dv["b"], dv["sb"], o0, dv["m_indices"])
    dg.dg_m_grouped_gemm_fp8_contiguous_fmt(dv["a"], dv["sa"], dv["b"], dv["sb"], o1, dv["m_indices"],
                                            a_fmt="e4m3", b_fmt="e4m3")
    md = W.make_masked(3, 64, 96, 256, seed=34, masked_m=[64, 0, 9])
    mv = upload(md)
    p0, p1 = sentinel_like((3, 64, 96)), sentinel_like((3, 64, 96))
    dg.dg_m_grouped_gemm_fp8_masked(mv["a"], mv["sa"], mv["b"], mv["sb"], p0, mv["masked_m"])
    dg.dg_m_grouped_gemm_fp8_masked_fmt(mv["a"], mv["sa"], mv["b"], mv["sb"], p1, mv["masked_m"],
                                        a_fmt="e4m3", b_fmt="e4m3")
    torch.cuda.synchronize()
    assert np.array_equal(bits(o0), bits(o1))
    assert np.array_equal(bits(p0), bits(p1))


def test_grouped_forced_config_without_formats_is_unsupported():
    plain = [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 2 and not c["all_formats"]]
    assert plain
    md = W.make_masked(2, 64, 96, 256, seed=35, masked_m=[64, 9], a_fmt="e5m2", b_fmt="e5m2")
    with pytest.raises(dg.DGError) as e:
        run_masked_fmt(md, plain[0])
    assert e.value.status == dg.DG_ERR_UNSUPPORTED
