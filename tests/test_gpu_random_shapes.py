"""Seeded random shapes on every layout, against the oracle.

Beyond the hand-picked edge shapes: M, N (multiples of 16) and K (multiples of 128)
drawn at random from a fixed seed, group counts and masked counts likewise, each run
through the planner and with one compiled configuration of the layout pinned (also
drawn), with a random CU cap for half of the cases.  Every valid row is compared with
the oracle; untouched rows and columns past N keep the sentinel bit for bit, and the
planned and pinned outputs are identical.
"""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu
CASES = 10


@pytest.fixture(scope="module", autouse=True)
def gpu():
    dev = require_gpu()
    dg.load_library()
    yield dev
    dg.dg_set_kernel_config(-1)
    dg.dg_set_num_cus(0)


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def configs_of(layout):
    return [c["id"] for c in dg.dg_kernel_config_info() if c["layout"] == layout]


def run(call, cfg, cap):
    import torch
    dg.dg_set_num_cus(cap)
    dg.dg_set_kernel_config(cfg)
    try:
        call()
        torch.cuda.synchronize()
    finally:
        dg.dg_set_kernel_config(-1)
        dg.dg_set_num_cus(0)


@pytest.mark.parametrize("case", range(CASES))
def test_dense_random(orc, case):
    rng = np.random.default_rng(1000 + case)
    m = int(rng.integers(1, 700))
    n = 16 * int(rng.integers(1, 60))
    k = 128 * int(rng.integers(1, 13))
    cfg = int(rng.choice(configs_of(0)))
    cap = int(rng.choice([0, 0, 5, 37, 200]))
    dd = W.make_dense(m, n, k, seed=2000 + case)
    dv = {x: to_dev(dd[x]) for x in ("a", "sa", "b", "sb")}
    ref = orc.gemm_fp8_nt(dd["a"], dd["sa"], dd["b"], dd["sb"])
    outs = []
    for c in (-1, cfg):
        full = sentinel_like((m, n + 16))
        say(f"dense random case {case}: {m}x{n}x{k} cfg={c} cap={cap}")
        run(lambda: dg.dg_gemm_fp8_nt(dv["a"], dv["sa"], dv["b"], dv["sb"], full[:, :n]), c, cap)
        fb = bits(full)
        assert np.all(fb[:, n:] == W.SENTINEL_BF16), "a column past N was written"
        check_values(fb[:, :n], ref, f"dense {m}x{n}x{k} cfg{c}")
        outs.append(fb)
    # bit-identical where both sum every K block in one chain (every configuration but
    # the K-group ones, which add two partial sums at the end)
    planned = dg.dg_describe_launch(0, m, n, k, 1, cap)["config_id"]
    groups = {c["id"]: c["k_groups"] for c in dg.dg_kernel_config_info()}
    if groups[planned] == groups[cfg]:
        assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("case", range(CASES))
def test_contiguous_random(orc, case):
    rng = np.random.default_rng(3000 + case)
    groups = int(rng.integers(1, 7))
    counts = [int(c) for c in rng.integers(0, 400, groups)]
    n = 16 * int(rng.integers(1, 40))
    k = 128 * int(rng.integers(1, 9))
    cfg = int(rng.choice(configs_of(1)))
    cap = int(rng.choice([0, 0, 7, 64]))
    cd = W.make_contiguous(counts, n=n, k=k, seed=4000 + case)
    if cd["m_total"] == 0:
        pytest.skip("all groups empty")
    dv = {x: to_dev(cd[x]) for x in ("a", "sa", "b", "sb", "m_indices")}
    sentinel = np.full((cd["m_total"], n), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel)
    valid = cd["m_indices"] >= 0
    outs = []
    for c in (-1, cfg):
        out = sentinel_like((cd["m_total"], n))
        say(f"contiguous random case {case}: counts={counts} n={n} k={k} cfg={c} cap={cap}")
        run(lambda: dg.dg_m_grouped_gemm_fp8_contiguous(dv["a"], dv["sa"], dv["b"], dv["sb"], out,
                                                        dv["m_indices"]), c, cap)
        ob = bits(out)
        assert np.all(ob[~valid] == W.SENTINEL_BF16), "a padding row was written"
        if valid.any():
            check_values(ob[valid], ref[valid], f"contiguous counts={counts} cfg{c}")
        outs.append(ob)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("case", range(CASES))
def test_masked_random(orc, case):
    rng = np.random.default_rng(5000 + case)
    groups = int(rng.integers(1, 9))
    max_m = int(rng.integers(1, 300))
    mm = [int(v) for v in rng.integers(-2, max_m + 3, groups)]       # out-of-range counts included
    n = 16 * int(rng.integers(1, 40))
    k = 128 * int(rng.integers(1, 9))
    cfg = int(rng.choice(configs_of(2)))
    cap = int(rng.choice([0, 0, 9, 100]))
    md = W.make_masked(groups, max_m, n, k, seed=6000 + case, masked_m=mm)
    dv = {x: to_dev(md[x]) for x in ("a", "sa", "b", "sb", "masked_m")}
    clamped = np.clip(np.array(mm), 0, max_m)
    sentinel = np.full((groups, max_m, n), W.SENTINEL_BF16, np.uint16)
    ref = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], clamped, d_init=sentinel)
    valid = np.arange(max_m)[None, :] < clamped[:, None]
    outs = []
    for c in (-1, cfg):
        out = sentinel_like((groups, max_m, n))
        say(f"masked random case {case}: masked_m={mm} max_m={max_m} n={n} k={k} cfg={c} cap={cap}")
        run(lambda: dg.dg_m_grouped_gemm_fp8_masked(dv["a"], dv["sa"], dv["b"], dv["sb"], out, dv["masked_m"]),
            c, cap)
        ob = bits(out)
        assert np.all(ob[~valid] == W.SENTINEL_BF16), "a row at or past masked_m was written"
        if valid.any():
            check_values(ob[valid], ref[valid], f"masked masked_m={mm} cfg{c}")
        outs.append(ob)
    assert np.array_equal(outs[0], outs[1])
