"""Maximum sizes: operands larger than 4 GiB, on each layout.

The kernels address a tile through 32-bit buffer offsets from the tile's first row and
form the tile's (and the group's) base address in 64 bits; these tests put rows of A
past the 4 GiB byte offset and check them.  The operands are generated on the GPU with
a seeded generator (too large to build on the host); the rows checked are copied back
and compared with the oracle, chosen on both sides of the 4 GiB boundary, at tile
edges and at the last row.  Rows that must stay untouched (padding, rows at or past
masked_m) are checked against the sentinel.
"""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu

K = 7168
N = 128
KB = K // 128
FOUR_GIB = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def gpu():
    dev = require_gpu()
    dg.load_library()
    yield dev
    import torch
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def fp8_on_device(shape, seed):
    """Random E4M3 bytes with the two NaN codes replaced by 448, made on the GPU."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=gen)
    x.sub_(((x & 0x7F) == 0x7F).to(torch.uint8))     # 0x7F -> 0x7E, 0xFF -> 0xFE
    return x


def scales_on_device(shape, seed):
    import torch
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return torch.rand(shape, device="cuda", generator=gen) * 1.5 + 0.25


def b_operand(groups, seed):
    """B and sB of the shared generator ([groups][N][K], [groups][N/128][K/128])."""
    bs, sbs = [], []
    for g in range(groups):
        d = W.make_dense(16, N, K, seed=seed + g)
        bs.append(d["b"])
        sbs.append(d["sb"])
    return np.stack(bs), np.stack(sbs)


def rows_past(first_row_offset_rows, total_rows):
    """Rows on both sides of the first row that starts past 4 GiB, tile edges, the last row."""
    cut = -(-FOUR_GIB // K) - first_row_offset_rows        # first row whose bytes start past 4 GiB
    rows = {0, 255, 256, cut - 1, cut, cut + 1, total_rows // 2, total_rows - 257, total_rows - 256,
            total_rows - 1}
    return sorted(r for r in rows if 0 <= r < total_rows)


def test_dense_a_past_4gib(orc):
    import torch
    m = 600_064                                   # m * K = 4.3e9 bytes
    assert m * K > FOUR_GIB
    a = fp8_on_device((m, K), seed=101)
    sa = scales_on_device((KB, m), seed=102)
    b, sb = b_operand(1, seed=103)
    out = sentinel_like((m, N))
    say(f"dense {m}x{N}x{K}: A is {m * K / 2**30:.2f} GiB", dg.dg_describe_launch(0, m, N, K, 1))
    dg.dg_gemm_fp8_nt(a, sa, to_dev(b[0]), to_dev(sb[0]), out)
    torch.cuda.synchronize()
    rows = rows_past(0, m)
    idx = torch.tensor(rows, device="cuda")
    got = bits(out.index_select(0, idx))
    ref = orc.gemm_fp8_nt(a.index_select(0, idx).cpu().numpy(), sa.index_select(1, idx).cpu().numpy(), b[0], sb[0])
    check_values(got, ref, f"dense rows {rows}")
    del a, sa, out
    torch.cuda.empty_cache()


def test_contiguous_a_past_4gib(orc):
    import torch
    m_total = 600_064
    g0_rows, g0_pad = 299_990, 42                 # group 0, then 42 padding rows up to 300032
    mi = np.full(m_total, 1, np.int32)
    mi[:g0_rows] = 0
    mi[g0_rows:g0_rows + g0_pad] = -1
    assert dg.dg_check_contiguous_layout(mi, 2) is None
    a = fp8_on_device((m_total, K), seed=111)
    sa = scales_on_device((KB, m_total), seed=112)
    b, sb = b_operand(2, seed=113)
    out = sentinel_like((m_total, N))
    say(f"contiguous {m_total}x{N}x{K}: A is {m_total * K / 2**30:.2f} GiB")
    dg.dg_m_grouped_gemm_fp8_contiguous(a, sa, to_dev(b), to_dev(sb), out, to_dev(mi))
    torch.cuda.synchronize()
    rows = sorted(set(rows_past(0, m_total)) | {g0_rows - 1, g0_rows, g0_rows + g0_pad - 1, g0_rows + g0_pad})
    idx = torch.tensor(rows, device="cuda")
    got = bits(out.index_select(0, idx))
    a_rows = a.index_select(0, idx).cpu().numpy()
    sa_rows = sa.index_select(1, idx).cpu().numpy()
    for i, r in enumerate(rows):
        g = mi[r]
        if g < 0:
            assert np.all(got[i] == W.SENTINEL_BF16), f"padding row {r} was written"
            continue
        ref = orc.gemm_fp8_nt(a_rows[i:i + 1], sa_rows[:, i:i + 1], b[g], sb[g])
        check_values(got[i:i + 1], ref, f"contiguous row {r} (group {g})")
    del a, sa, out
    torch.cuda.empty_cache()


def test_masked_a_past_4gib(orc):
    import torch
    groups, max_m = 2, 300_032
    assert groups * max_m * K > FOUR_GIB
    mm = np.array([77, max_m], np.int32)
    a = fp8_on_device((groups, max_m, K), seed=121)
    sa = scales_on_device((groups, KB, max_m), seed=122)
    b, sb = b_operand(groups, seed=123)
    out = sentinel_like((groups, max_m, N))
    say(f"masked {groups}x{max_m}x{N}x{K}: A is {groups * max_m * K / 2**30:.2f} GiB")
    dg.dg_m_grouped_gemm_fp8_masked(a, sa, to_dev(b), to_dev(sb), out, to_dev(mm))
    torch.cuda.synchronize()
    # group 0: every valid row, and untouched rows past masked_m
    idx0 = torch.arange(0, 77, device="cuda")
    got0 = bits(out[0].index_select(0, idx0))
    ref0 = orc.gemm_fp8_nt(a[0, :77].cpu().numpy(), np.ascontiguousarray(sa[0, :, :77].cpu().numpy()), b[0], sb[0])
    check_values(got0, ref0, "masked group 0")
    assert np.all(bits(out[0, 77:1000]) == W.SENTINEL_BF16)
    assert np.all(bits(out[0, max_m - 300:]) == W.SENTINEL_BF16)
    # group 1 starts at max_m * K bytes: its rows cross 4 GiB
    rows = rows_past(max_m, max_m)
    idx = torch.tensor(rows, device="cuda")
    got = bits(out[1].index_select(0, idx))
    ref = orc.gemm_fp8_nt(a[1].index_select(0, idx).cpu().numpy(), sa[1].index_select(1, idx).cpu().numpy(),
                          b[1], sb[1])
    check_values(got, ref, f"masked group 1 rows {rows}")
    del a, sa, out
    torch.cuda.empty_cache()
