"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Every output is compared element by element with the oracle over all of its valid
rows: small and ragged shapes on every compiled configuration, and the full-size
workloads in the launch configuration the bench times.  Whole-output properties
are checked bit-exactly as well: no NaN/Inf, untouched padding / masked rows,
nothing written past column N, grouped output equal to the dense kernel's output
per group.
"""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, say, sentinel_like, to_dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    dev = require_gpu()
    dg.load_library()
    yield dev
    dg.dg_set_kernel_config(-1)
    dg.dg_set_num_cus(0)


def configs_of(layout):
    return [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == layout]


def k_groups(cfg, m=0, n=0, k=0):
    """Summation class of a configuration: 1 = one promotion chain over all K blocks
    (every such configuration gives the same bits), 2 = two wave groups over alternate
    K blocks whose sums are added at the end (the same bits as each other, not as
    class 1).  cfg -1 is the planner's pick for a dense m x n x k call."""
    if cfg == -1:
        cfg = dg.dg_describe_launch(0, m, n, k, 1)["config_id"]
    return {c["id"]: c["k_groups"] for c in dg.dg_kernel_config_info()}[cfg]


def assert_equal_per_class(outs):
    """outs: [(summation class, bits)]; the outputs of one class are identical."""
    first = {}
    for cls, o in outs:
        if cls in first:
            assert np.array_equal(o, first[cls]), f"outputs of summation class {cls} differ"
        else:
            first[cls] = o


# a dense configuration with one promotion chain, for bit-exact comparisons with the
# grouped layouts (which sum every K block in one chain)
def dense_one_chain():
    return next(c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 0 and c["k_groups"] == 1)


def run_dense(dd, cfg=-1, pad_cols=16):
    """GPU dense GEMM into a sentinel-filled buffer wider than N; returns (out bits, full bits)."""
    import torch
    dv = upload(dd)
    m, n = dd["a"].shape[0], dd["b"].shape[0]
    full = sentinel_like((m, n + pad_cols))
    dg.dg_set_kernel_config(cfg)
    dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], full[:, :n])
    torch.cuda.synchronize()
    dg.dg_set_kernel_config(-1)
    fb = bits(full)
    return fb[:, :n], fb


def oracle_dense(orc, dd, rows=None):
    a, sa = dd["a"], dd["sa"]
    if rows is not None:
        a, sa = a[rows], sa[:, rows]
    return orc.gemm_fp8_nt(a, sa, dd["b"], dd["sb"])


# --------------------------------------------------------------------------- dense
def test_dense_small_workload_all_configs(orc):
    dd = W.make(W.WORKLOADS["dense_m128_n128_k512"])
    ref = oracle_dense(orc, dd)
    outs = []
    for cfg in [-1] + configs_of(0):
        say(f"dense 128x128x512 cfg={cfg}")
        out, full = run_dense(dd, cfg)
        check_values(out, ref, f"dense128 cfg{cfg}")
        assert np.all(full[:, 128:] == W.SENTINEL_BF16)
        outs.append((k_groups(cfg, 128, 128, 512), out))
    assert_equal_per_class(outs)                   # identical arithmetic in every tile shape


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (17, 48, 256), (300, 208, 384), (129, 400, 640),
                                   (513, 1040, 1024), (64, 7168 // 4, 128)])
def test_dense_ragged_shapes(orc, m, n, k):
    dd = W.make_dense(m, n, k, seed=m + n + k)
    ref = oracle_dense(orc, dd)
    outs = []
    for cfg in configs_of(0):
        say(f"dense ragged m={m} n={n} k={k} cfg={cfg}")
        out, full = run_dense(dd, cfg)
        check_values(out, ref, f"dense {m}x{n}x{k} cfg{cfg}")
        assert np.all(full[:, n:] == W.SENTINEL_BF16), "wrote past column n"
        outs.append((k_groups(cfg), out))
    assert_equal_per_class(outs)


@pytest.mark.parametrize("m,n,k", [(300, 400, 640), (64, 7168, 2048)])
def test_dense_strided_operands(orc, m, n, k):
    """A, B, sA and D as views into wider buffers (row strides lda = K + 256, ldb = K + 128,
    ld_sa = the aligned M + 8, ldd = N + 24): the same bits as with packed operands on
    every configuration, the oracle's values, and nothing written between rows."""
    import torch
    dd = W.make_dense(m, n, k, seed=m + n + k)
    ref = oracle_dense(orc, dd)
    packed = {}
    for cls in (1, 2):
        cfg = next(c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 0 and c["k_groups"] == cls)
        packed[cls], _ = run_dense(dd, cfg)
        check_values(packed[cls], ref, f"dense packed {m}x{n}x{k} cfg{cfg}")
    lda, ldb, ld_sa, ldd = k + 256, k + 128, dd["sa"].shape[1] + 8, n + 24
    a_buf = torch.zeros((m, lda), dtype=torch.uint8, device="cuda:0")
    b_buf = torch.zeros((n, ldb), dtype=torch.uint8, device="cuda:0")
    sa_buf = torch.zeros((k // 128, ld_sa), dtype=torch.float32, device="cuda:0")
    a_buf[:, :k] = to_dev(dd["a"])
    b_buf[:, :k] = to_dev(dd["b"])
    sa_buf[:, :dd["sa"].shape[1]] = to_dev(dd["sa"])
    sb = to_dev(dd["sb"])
    for cfg in [-1] + configs_of(0):
        d_buf = sentinel_like((m, ldd))
        say(f"dense strided {m}x{n}x{k} cfg={cfg}")
        dg.dg_set_kernel_config(cfg)
        try:
            dg.dg_gemm_fp8_nt(a_buf[:, :k], sa_buf[:, :m], b_buf[:, :k], sb, d_buf[:, :n])
            torch.cuda.synchronize()
        finally:
            dg.dg_set_kernel_config(-1)
        fb = bits(d_buf)
        assert np.array_equal(fb[:, :n], packed[k_groups(cfg, m, n, k)]), \
            f"strided operands changed the result (cfg {cfg})"
        assert np.all(fb[:, n:] == W.SENTINEL_BF16), "a column between rows was written"


def test_dense_under_filled_workload_full_compare(orc):
    dd = W.make(W.WORKLOADS["dense_m256_n7168_k2048"])
    say("dense 256x7168x2048 (planned config)", dg.dg_describe_launch(0, 256, 7168, 2048, 1))
    out, _ = run_dense(dd)
    ref = oracle_dense(orc, dd)
    check_values(out, ref, "dense 256x7168x2048")


def test_dense_prefill_workload_full_compare(orc):
    dd = W.make(W.WORKLOADS["dense_m4096_n7168_k7168"])
    say("dense 4096x7168x7168 (planned config)", dg.dg_describe_launch(0, 4096, 7168, 7168, 1))
    out, full = run_dense(dd)
    assert np.all(full[:, 7168:] == W.SENTINEL_BF16)
    assert not np.any(out == W.SENTINEL_BF16)
    say("dense 4096x7168x7168: oracle over all rows")
    check_values(out, oracle_dense(orc, dd), "dense 4096x7168x7168 all rows")


def test_dense_cu_cap_is_bit_identical(orc):
    dd = W.make_dense(512, 1024, 512, seed=77)
    base, _ = run_dense(dd)
    for cap in (37, 64):
        dg.dg_set_num_cus(cap)
        say(f"dense 512x1024x512 with cu cap {cap}")
        out, _ = run_dense(dd)
        dg.dg_set_num_cus(0)
        assert np.array_equal(out, base)
    check_values(base, oracle_dense(orc, dd), "dense 512x1024x512")


@pytest.mark.parametrize("k", [512, 640, 768])
def test_dense_chained_tiles_all_configs(orc, k):
    """Three workgroups, many tiles each: where K/128 splits into whole groups of a
    config's LDS stages, each tile's last blocks already fetch the next tile's first
    ones.  Ragged M and N put partial tiles and idle waves into the chains."""
    dd = W.make_dense(300, 464, k, seed=k + 5)
    ref = oracle_dense(orc, dd)
    dg.dg_set_num_cus(3)
    try:
        for cfg in configs_of(0):
            say(f"dense 300x464x{k} cfg={cfg} cu cap 3")
            out, full = run_dense(dd, cfg)
            check_values(out, ref, f"dense 300x464x{k} cfg{cfg} chained")
            assert np.all(full[:, 464:] == W.SENTINEL_BF16)
    finally:
        dg.dg_set_num_cus(0)


@pytest.mark.parametrize("k", [7168, 2048])
def test_dense_shape_instances(orc, k):
    """N = 7168 with K = 7168 or K = 2048 runs the instances compiled for that shape in
    the configurations that have them: their output equals the generic
    configurations' bit for bit and the oracle, on one tile per workgroup and on three
    workgroups chaining tiles."""
    dd = W.make_dense(300, 7168, k, seed=k + 9)
    ref = oracle_dense(orc, dd)
    specs = [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 0 and c["shape_specialised"]]
    generic = [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == 0 and not c["shape_specialised"]]
    assert specs and generic
    base, _ = run_dense(dd, generic[0])
    check_values(base, ref, f"dense 300x7168x{k} generic cfg{generic[0]}")
    try:
        for cap in (0, 3):
            dg.dg_set_num_cus(cap)
            for cfg in specs:
                say(f"dense 300x7168x{k} cfg={cfg} (shape instance) cu cap {cap}")
                out, full = run_dense(dd, cfg)
                assert np.array_equal(out, base), f"cfg{cfg} cap {cap} differs from the generic kernel"
                assert np.all(full[:, 7168:] == W.SENTINEL_BF16)
    finally:
        dg.dg_set_num_cus(0)


@pytest.mark.parametrize("m,n,k", [(64, 4096, 7168), (128, 2048, 4096)])
def test_dense_k_groups_planned_full_compare(orc, m, n, k):
    """Under-filled long-K shapes plan two wave groups over alternate K blocks: the
    whole output against the oracle, and within the same tolerance of a one-chain
    configuration's output (the two differ only in how the K blocks' sums are
    rounded together)."""
    d = dg.dg_describe_launch(0, m, n, k, 1)
    assert k_groups(d["config_id"]) == 2, d
    dd = W.make_dense(m, n, k, seed=m + k)
    ref = oracle_dense(orc, dd)
    say(f"dense {m}x{n}x{k} planned cfg={d['config_id']}")
    out, full = run_dense(dd)
    assert np.all(full[:, n:] == W.SENTINEL_BF16)
    check_values(out, ref, f"dense {m}x{n}x{k} k groups")
    one, _ = run_dense(dd, dense_one_chain())
    check_values(one, ref, f"dense {m}x{n}x{k} one chain")


def test_dense_k_groups_deterministic():
    """The two-K-group configuration adds its groups' sums in a fixed order: the same bits
    under CU caps (fewer workgroups, more tiles each) and in every replay of a captured
    HIP graph, with eager work between the replays."""
    import torch
    m, n, k = 64, 2048, 4096
    cfg = dg.dg_describe_launch(0, m, n, k, 1)["config_id"]
    assert k_groups(cfg) == 2
    dd = W.make_dense(m, n, k, seed=57)
    base, _ = run_dense(dd)
    for cap in (37, 5):
        dg.dg_set_num_cus(cap)
        try:
            say(f"dense {m}x{n}x{k} cfg={cfg}, cu cap {cap}")
            out, _ = run_dense(dd, cfg)
        finally:
            dg.dg_set_num_cus(0)
        assert np.array_equal(out, base), f"cu cap {cap} changed the bits"
    dv = upload(dd)
    d = sentinel_like((m, n))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):      # warm-up outside capture
        dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], d)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], d)
    for rep in range(3):
        d.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"dense {m}x{n}x{k} k groups, graph replay {rep}")
        assert np.array_equal(bits(d), base), f"replay {rep} differs from the eager call"


def test_dense_per_tensor_scaling(orc):
    """Per-tensor scaling is the special case of one value in every scale block: the
    same kernel, checked against the oracle with constant sA and sB."""
    dd = W.make_dense(384, 640, 1024, seed=31)
    dd["sa"] = np.full_like(dd["sa"], 0.0078125 * 3)
    dd["sb"] = np.full_like(dd["sb"], 1.5)
    out, _ = run_dense(dd)
    check_values(out, oracle_dense(orc, dd), "dense per-tensor scales")


# --------------------------------------------------------------------------- contiguous
def run_contiguous(cd, cfg=-1):
    import torch
    dv = upload(cd)
    out = sentinel_like((cd["m_total"], cd["n"]))
    dg.dg_set_kernel_config(cfg)
    dg.dg_m_grouped_gemm_fp8_contiguous(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["m_indices"])
    torch.cuda.synchronize()
    dg.dg_set_kernel_config(-1)
    return bits(out)


def dense_gpu_segment(cd, g, lo, hi):
    """The dense kernel on one group's rows (its own call) for bit-exact comparison."""
    seg = {"a": cd["a"][lo:hi], "sa": np.ascontiguousarray(cd["sa"][:, lo:hi]), "b": cd["b"][g],
           "sb": cd["sb"][g]}
    seg["sa"] = np.pad(seg["sa"], ((0, 0), (0, (-seg["sa"].shape[1]) % 4)))
    out, _ = run_dense(seg, dense_one_chain())
    return out


def test_contiguous_small_all_configs(orc):
    counts = [130, 0, 1, 257, 128]
    cd = W.make_contiguous(counts, n=272, k=384, seed=21)
    sentinel = np.full((cd["m_total"], 272), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    valid = cd["m_indices"] >= 0
    outs = []
    for cfg in configs_of(1):
        say(f"contiguous small counts={counts} cfg={cfg}")
        out = run_contiguous(cd, cfg)
        check_values(out[valid], ref[valid], f"contiguous small cfg{cfg}")
        assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    off = 0
    for g, (c, p) in enumerate(zip(counts, W.padded(counts))):
        if c:
            assert np.array_equal(dense_gpu_segment(cd, g, off, off + c), outs[0][off:off + c])
        off += p


@pytest.mark.parametrize("k", [512, 768])
def test_contiguous_chained_tiles_all_configs(orc, k):
    """Contiguous layout with three workgroups: chains of tiles that mix one-group tiles,
    two-group tiles (two passes) and padding, with and without next-tile prefetch."""
    counts = [130, 0, 1, 257, 128, 40]
    cd = W.make_contiguous(counts, n=400, k=k, seed=k + 9)
    sentinel = np.full((cd["m_total"], 400), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    valid = cd["m_indices"] >= 0
    dg.dg_set_num_cus(3)
    try:
        for cfg in configs_of(1):
            say(f"contiguous counts={counts} k={k} cfg={cfg} cu cap 3")
            out = run_contiguous(cd, cfg)
            check_values(out[valid], ref[valid], f"contiguous k={k} cfg{cfg} chained")
            assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
    finally:
        dg.dg_set_num_cus(0)


def test_contiguous_workload_full_compare(orc):
    w = W.WORKLOADS["contiguous_g8_t32768_zipf1.1_n4096_k7168"]
    cd = W.make(w)
    say("contiguous 8x4096x7168 zipf (planned config)",
        dg.dg_describe_launch(1, cd["m_total"], 4096, 7168, 8))
    out = run_contiguous(cd)
    valid = cd["m_indices"] >= 0
    assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
    assert not np.any(out[valid] == W.SENTINEL_BF16), "a valid row was not written"
    say("contiguous 8x4096x7168 zipf: oracle over all valid rows")
    sentinel = np.full(out.shape, W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    check_values(out[valid], ref[valid], "contiguous workload all valid rows")
    # grouped == dense per group, bit for bit, on every group
    off = 0
    for g, (c, p) in enumerate(zip(cd["counts"], W.padded(cd["counts"]))):
        say(f"contiguous workload: group {g} ({c} rows) against the dense kernel")
        assert np.array_equal(dense_gpu_segment(cd, g, off, off + c), out[off:off + c]), f"group {g}"
        off += p


def test_contiguous_shape_instance_all_configs(orc):
    """N = 4096 with K = 7168 runs the instance compiled for that shape in the contiguous
    configurations that have one: every contiguous configuration gives the same bits,
    within tolerance of the oracle, with one tile per workgroup and with three
    workgroups chaining tiles (two-group tiles and padding included)."""
    counts = [130, 0, 257, 40]
    cd = W.make_contiguous(counts, n=4096, k=7168, seed=61)
    assert any(c["shape_specialised"] for c in dg.dg_kernel_config_info() if c["layout"] == 1)
    sentinel = np.full((cd["m_total"], 4096), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    valid = cd["m_indices"] >= 0
    outs = []
    try:
        for cap in (0, 3):
            dg.dg_set_num_cus(cap)
            for cfg in configs_of(1):
                say(f"contiguous counts={counts} n=4096 k=7168 cfg={cfg} cu cap {cap}")
                out = run_contiguous(cd, cfg)
                assert np.all(out[~valid] == W.SENTINEL_BF16), "a padding row was written"
                outs.append(out)
    finally:
        dg.dg_set_num_cus(0)
    check_values(outs[0][valid], ref[valid], "contiguous n=4096 k=7168")
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_contiguous_rows_breaking_the_block_rule_are_not_written(orc):
    """m_indices that break the layout's precondition (an entry naming another group or
    an out-of-range group inside a 128-row block): the call computes each block for the
    group of its first row and writes only the rows that carry that group, so the
    offending rows keep their previous contents; the others are exact."""
    counts = [200, 130, 60]
    cd = W.make_contiguous(counts, n=144, k=256, seed=51)
    mi = cd["m_indices"].copy()
    mi[5] = 1            # group 0's first block: a row naming group 1
    mi[140] = 2          # group 0's second block (rows 128..199 valid)
    mi[300] = 9          # group 1's second block: out of range
    mi[260] = -1         # padding inside group 1's rows (allowed)
    assert dg.dg_check_contiguous_layout(mi, 3) == 5
    cd2 = dict(cd, m_indices=mi)
    for cfg in configs_of(1):
        say(f"contiguous with broken blocks cfg={cfg}")
        out = run_contiguous(cd2, cfg)
        keep = np.zeros(cd["m_total"], bool)
        for b in range(0, cd["m_total"], 128):
            keep[b:b + 128] = mi[b:b + 128] == mi[b]
        keep &= mi >= 0
        assert np.all(out[~keep] == W.SENTINEL_BF16), f"cfg{cfg}: a row outside its block's group was written"
        sentinel = np.full(out.shape, W.SENTINEL_BF16, np.uint16)
        ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], np.where(keep, mi, -1),
                                       d_init=sentinel)
        check_values(out[keep], ref[keep], f"contiguous broken blocks cfg{cfg}")


# --------------------------------------------------------------------------- masked
def run_masked(md, cfg=-1, masked_m=None):
    import torch
    dv = upload(md)
    if masked_m is not None:
        dv["masked_m"] = to_dev(np.asarray(masked_m, np.int32))
    out = sentinel_like((md["groups"], md["max_m"], md["n"]))
    dg.dg_set_kernel_config(cfg)
    dg.dg_m_grouped_gemm_fp8_masked(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"])
    torch.cuda.synchronize()
    dg.dg_set_kernel_config(-1)
    return bits(out)


def check_masked(orc, md, out):
    """Rows >= masked_m untouched and every valid row written (bit-exact), every valid
    row of every group within tolerance of the oracle (one call's valid rows together)."""
    mm = np.clip(md["masked_m"], 0, md["max_m"])
    for g in range(md["groups"]):
        assert np.all(out[g, mm[g]:] == W.SENTINEL_BF16), f"group {g}: a row >= masked_m was written"
        assert not np.any(out[g, :mm[g]] == W.SENTINEL_BF16), f"group {g}: a valid row was not written"
    if mm.sum() == 0:
        return
    sentinel = np.full(out.shape, W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], mm, d_init=sentinel)
    valid = np.arange(md["max_m"])[None, :] < mm[:, None]
    check_values(out[valid], ref[valid], "masked, all valid rows")


@pytest.mark.parametrize("max_m", [256, 70])
def test_masked_edges_all_configs(orc, max_m):
    mm = [0, max_m, 1, max_m - 1, 16, 17, min(128, max_m), min(129, max_m), 0, 33]
    md = W.make_masked(len(mm), max_m, 272, 256, seed=31, masked_m=mm)
    outs = []
    for cfg in configs_of(2):
        say(f"masked edges max_m={max_m} cfg={cfg}")
        out = run_masked(md, cfg)
        check_masked(orc, md, out)
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    for g in (1, 3, 5):
        seg = {"a": md["a"][g][:mm[g]], "sa": md["sa"][g][:, :mm[g]], "b": md["b"][g], "sb": md["sb"][g]}
        seg["sa"] = np.pad(seg["sa"], ((0, 0), (0, (-mm[g]) % 4)))
        dense, _ = run_dense(seg, dense_one_chain())
        assert np.array_equal(dense, outs[0][g, :mm[g]])


def test_masked_capacity_beyond_one_row_block(orc):
    """A capacity of 600 rows spans three 256-row blocks (and five 128-row ones): counts
    at and around the block edges, every masked configuration bit-identical, within
    tolerance of the oracle, rows at or past masked_m untouched."""
    mm = [0, 600, 1, 255, 256, 257, 511, 512, 599, 384]
    md = W.make_masked(len(mm), 600, 144, 384, seed=71, masked_m=mm)
    outs = []
    for cfg in configs_of(2):
        say(f"masked capacity 600 counts={mm} cfg={cfg}")
        out = run_masked(md, cfg)
        check_masked(orc, md, out)
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_masked_shape_instance_all_configs(orc):
    """N = 4096 with K = 7168 runs the instance compiled for that shape in the masked
    configurations that have one: every masked configuration gives the same bits,
    within tolerance of the oracle, with one tile per workgroup and with three
    workgroups chaining tiles."""
    mm = [0, 256, 77, 129]
    md = W.make_masked(len(mm), 256, 4096, 7168, seed=62, masked_m=mm)
    assert any(c["shape_specialised"] for c in dg.dg_kernel_config_info() if c["layout"] == 2)
    outs = []
    try:
        for cap in (0, 3):
            dg.dg_set_num_cus(cap)
            for cfg in configs_of(2):
                say(f"masked counts={mm} n=4096 k=7168 cfg={cfg} cu cap {cap}")
                outs.append(run_masked(md, cfg))
    finally:
        dg.dg_set_num_cus(0)
    check_masked(orc, md, outs[0])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_masked_out_of_range_counts_are_clamped(orc):
    md = W.make_masked(3, 64, 128, 128, seed=32, masked_m=[-3, 500, 5])
    out = run_masked(md)
    assert np.all(out[0] == W.SENTINEL_BF16)
    md2 = dict(md, masked_m=np.array([0, 64, 5], np.int32))
    check_masked(orc, md2, out)


def test_masked_all_empty_is_noop():
    md = W.make_masked(4, 256, 128, 128, seed=33, masked_m=[0, 0, 0, 0])
    out = run_masked(md)
    assert np.all(out == W.SENTINEL_BF16)


def test_masked_workload_full_compare(orc):
    md = W.make(W.WORKLOADS["masked_g16_cap256_n4096_k7168"])
    say("masked 16x256x4096x7168 masked_m=", md["masked_m"].tolist(),
        dg.dg_describe_launch(2, 256, 4096, 7168, 16))
    out = run_masked(md)
    check_masked(orc, md, out)


def test_masked_graph_replay_reads_device_counts(orc):
    """The masked call captured once in a graph follows masked_m changed on the device
    between replays (the host never reads it)."""
    import torch
    md = W.make_masked(6, 128, 256, 256, seed=34, masked_m=[5, 0, 128, 64, 1, 100])
    dv = upload(md)
    out = sentinel_like((6, 128, 256))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):      # warm-up outside capture
        dg.dg_m_grouped_gemm_fp8_masked(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.dg_m_grouped_gemm_fp8_masked(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"])
    for counts in ([5, 0, 128, 64, 1, 100], [128, 3, 0, 17, 128, 0], [1, 1, 1, 1, 1, 1]):
        say(f"graph replay masked_m={counts}")
        out.fill_(W.SENTINEL_BF16)
        dv["masked_m"].copy_(torch.tensor(counts, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out)
        eager = run_masked(md, masked_m=counts)
        assert np.array_equal(got, eager)
        check_masked(orc, dict(md, masked_m=np.array(counts, np.int32)), got)


def test_masked_maximum_group_count(orc):
    """1024 groups, the most the masked call takes (the device-side tile enumeration
    keeps a prefix over the groups in LDS), every count from 0 to the capacity."""
    groups, cap = 1024, 32
    mm = [int(x) for x in np.random.default_rng(46).integers(0, cap + 1, size=groups)]
    mm[0], mm[-1] = cap, cap
    md = W.make_masked(groups, cap, 32, 256, seed=46, masked_m=mm)
    say(f"masked {groups} groups, capacity {cap}, n=32 k=256")
    out = run_masked(md)
    sentinel = np.full(out.shape, W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], md["masked_m"], d_init=sentinel)
    for g in range(groups):
        assert np.all(out[g, mm[g]:] == W.SENTINEL_BF16), f"group {g}: a row >= masked_m was written"
    valid = np.concatenate([out[g, :mm[g]] for g in range(groups)])
    valid_ref = np.concatenate([ref[g, :mm[g]] for g in range(groups)])
    check_values(valid, valid_ref, "masked 1024 groups")


def test_contiguous_many_small_groups(orc):
    """300 experts with 0..40 tokens each: most 128-row blocks hold one small segment
    and its padding."""
    counts = [int(x) for x in np.random.default_rng(47).integers(0, 41, size=300)]
    cd = W.make_contiguous(counts, n=48, k=256, seed=47)
    say(f"contiguous 300 groups, m_total {cd['m_total']}, n=48 k=256")
    sentinel = np.full((cd["m_total"], 48), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    valid = cd["m_indices"] >= 0
    out = run_contiguous(cd)
    check_values(out[valid], ref[valid], "contiguous 300 groups")
    assert np.all(out[~valid] == W.SENTINEL_BF16)


def test_dense_and_contiguous_graph_replays_match_eager(orc):
    """Dense and contiguous calls captured into one graph give, on every replay (with
    eager work and synchronisation between replays and the inputs changed on the
    device in between), the eager calls' output bit for bit."""
    import torch
    dd = W.make_dense(320, 464, 512, seed=41)
    cd = W.make_contiguous([200, 5, 130], n=208, k=384, seed=42)
    dv, cv = upload(dd), upload(cd)
    od, oc = sentinel_like((320, 464)), sentinel_like((cd["m_total"], 208))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):      # warm-up outside capture
        dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], od)
        dg.dg_m_grouped_gemm_fp8_contiguous(cv["a"], cv["sa"], cv["b"], cv["sb"], oc, cv["m_indices"])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], od)
        dg.dg_m_grouped_gemm_fp8_contiguous(cv["a"], cv["sa"], cv["b"], cv["sb"], oc, cv["m_indices"])
    valid = cd["m_indices"] >= 0
    for rep in range(3):
        say(f"graph replay dense + contiguous, replay {rep}")
        if rep == 2:                      # new operands, written on the device
            dd = W.make_dense(320, 464, 512, seed=43)
            for key in ("a", "sa", "b", "sb"):
                dv[key].copy_(torch.from_numpy(dd[key]))
        od.fill_(W.SENTINEL_BF16)
        oc.fill_(W.SENTINEL_BF16)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_d, got_c = bits(od), bits(oc)
        eager_d, _ = run_dense(dd, pad_cols=0)
        eager_c = run_contiguous(cd)
        assert np.array_equal(got_d, eager_d), f"dense replay {rep} differs from the eager call"
        assert np.array_equal(got_c, eager_c), f"contiguous replay {rep} differs from the eager call"
        assert np.all(got_c[~valid] == W.SENTINEL_BF16)
    check_values(got_d, oracle_dense(orc, dd), "dense after graph replays")


def test_concurrent_streams_independent(orc):
    """Calls on two streams run concurrently (each grid fills the GPU, so they interleave
    on the hardware) and each result equals that call run alone."""
    import torch
    d1 = W.make_dense(1024, 2048, 1024, seed=44)
    d2 = W.make_dense(512, 4096, 2048, seed=45)
    alone1, _ = run_dense(d1, pad_cols=0)
    alone2, _ = run_dense(d2, pad_cols=0)
    v1, v2 = upload(d1), upload(d2)
    o1, o2 = sentinel_like((1024, 2048)), sentinel_like((512, 4096))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            dg.dg_gemm_fp8_nt(v1["a"], v1["sa"], v1["b"], v1["sb"], o1, stream=s1)
        with torch.cuda.stream(s2):
            dg.dg_gemm_fp8_nt(v2["a"], v2["sa"], v2["b"], v2["sb"], o2, stream=s2)
    torch.cuda.synchronize()
    say("two streams: 1024x2048x1024 and 512x4096x2048")
    assert np.array_equal(bits(o1), alone1)
    assert np.array_equal(bits(o2), alone2)
    check_values(alone1, oracle_dense(orc, d1), "stream 1 alone")


# --------------------------------------------------------------------------- errors
def test_binding_reports_validation_errors():
    import torch
    a = torch.zeros((64, 200), dtype=torch.uint8, device="cuda:0")
    b = torch.zeros((64, 200), dtype=torch.uint8, device="cuda:0")
    sa = torch.ones((2, 64), device="cuda:0")
    sb = torch.ones((1, 2), device="cuda:0")
    d = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(dg.DGError) as e:
        dg.dg_gemm_fp8_nt(a, sa, b, sb, d)
    assert e.value.status == dg.DG_ERR_UNSUPPORTED
    assert torch.count_nonzero(d).item() == 0


# --------------------------------------------------------------------------- seeded sweep
def test_seeded_random_shapes_planned(orc):
    """A fixed-seed sweep of ragged shapes, group counts and CU caps through the planner
    (whatever configuration, raster and variant it picks), each output compared in full."""
    rng = np.random.default_rng(2024)
    try:
        for i in range(10):
            m, n, k = int(rng.integers(1, 700)), 16 * int(rng.integers(1, 40)), 128 * int(rng.integers(1, 9))
            cap = int(rng.choice([0, 3, 17, 64, 200]))
            dg.dg_set_num_cus(cap)
            say(f"sweep dense {m}x{n}x{k} cap {cap}", dg.dg_describe_launch(0, m, n, k, 1))
            dd = W.make_dense(m, n, k, seed=100 + i)
            out, full = run_dense(dd)
            check_values(out, oracle_dense(orc, dd), f"sweep dense {m}x{n}x{k} cap {cap}")
            assert np.all(full[:, n:] == W.SENTINEL_BF16)
        for i in range(5):
            counts = [int(c) for c in rng.integers(0, 400, size=int(rng.integers(1, 7)))]
            n, k = 16 * int(rng.integers(1, 30)), 128 * int(rng.integers(1, 6))
            cap = int(rng.choice([0, 5, 48]))
            dg.dg_set_num_cus(cap)
            cd = W.make_contiguous(counts, n=n, k=k, seed=200 + i)
            say(f"sweep contiguous counts={counts} n={n} k={k} cap {cap}")
            sentinel = np.full((cd["m_total"], n), W.SENTINEL_BF16, np.uint16)
            ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
            valid = cd["m_indices"] >= 0
            out = run_contiguous(cd)
            check_values(out[valid], ref[valid], f"sweep contiguous {counts}")
            assert np.all(out[~valid] == W.SENTINEL_BF16)
        for i in range(5):
            groups, max_m = int(rng.integers(1, 9)), int(rng.choice([64, 128, 200, 256]))
            mm = [int(x) for x in rng.integers(0, max_m + 1, size=groups)]
            n, k = 16 * int(rng.integers(1, 30)), 128 * int(rng.integers(1, 6))
            cap = int(rng.choice([0, 7, 100]))
            dg.dg_set_num_cus(cap)
            md = W.make_masked(groups, max_m, n, k, seed=300 + i, masked_m=mm)
            say(f"sweep masked masked_m={mm} max_m={max_m} n={n} k={k} cap {cap}")
            check_masked(orc, md, run_masked(md))
    finally:
        dg.dg_set_num_cus(0)
