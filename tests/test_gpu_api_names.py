"""The README's Python names on the GPU: (data, scale) pairs with column-major LHS
scales made by get_col_major_tma_aligned_tensor, bit-identical to the dg_ calls they
marshal to, on each layout (row counts chosen so that the scales' leading dimension
is padded)."""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    yield require_gpu()


@pytest.fixture(scope="module")
def orc():
    import oracle
    return oracle


def col_major(sa_mn, rows):
    """MN-major [.., K/128, >= rows] -> row-major [.., rows, K/128] -> the README layout."""
    import torch
    rm = torch.from_numpy(np.ascontiguousarray(np.swapaxes(sa_mn[..., :rows], -1, -2))).cuda()
    cm = dg.get_col_major_tma_aligned_tensor(rm)
    assert tuple(cm.shape) == tuple(rm.shape)
    assert cm.stride(-2) == 1 and cm.stride(-1) == dg.get_tma_aligned_size(rows, 4)
    assert torch.equal(cm, rm)
    return cm


def test_gemm_fp8_fp8_bf16_nt(orc):
    import torch
    dd = W.make_dense(301, 272, 512, seed=81)
    dv = {k: to_dev(dd[k]) for k in ("a", "b", "sb")}
    sa_cm = col_major(dd["sa"], 301)
    out = sentinel_like((301, 272))
    say("gemm_fp8_fp8_bf16_nt 301x272x512")
    dg.gemm_fp8_fp8_bf16_nt((dv["a"], sa_cm), (dv["b"], dv["sb"]), out)
    ref_out = sentinel_like((301, 272))
    dg.dg_gemm_fp8_nt(dv["a"], to_dev(dd["sa"]), dv["b"], dv["sb"], ref_out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref_out))
    check_values(bits(out), orc.gemm_fp8_nt(dd["a"], dd["sa"], dd["b"], dd["sb"]), "gemm_fp8_fp8_bf16_nt")
    with pytest.raises(ValueError):
        dg.gemm_fp8_fp8_bf16_nt((dv["a"], sa_cm.contiguous()), (dv["b"], dv["sb"]), out)


def test_m_grouped_contiguous_names():
    import torch
    cd = W.make_contiguous([130, 0, 77], n=144, k=256, seed=82)
    dv = {k: to_dev(cd[k]) for k in ("a", "b", "sb", "m_indices")}
    sa_cm = col_major(cd["sa"], cd["m_total"])
    out, ref_out = sentinel_like((cd["m_total"], 144)), sentinel_like((cd["m_total"], 144))
    say("m_grouped_gemm_fp8_fp8_bf16_nt_contiguous")
    dg.m_grouped_gemm_fp8_fp8_bf16_nt_contiguous((dv["a"], sa_cm), (dv["b"], dv["sb"]), out, dv["m_indices"])
    dg.dg_m_grouped_gemm_fp8_contiguous(dv["a"], to_dev(cd["sa"]), dv["b"], dv["sb"], ref_out, dv["m_indices"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref_out))


def test_m_grouped_masked_names():
    import torch
    md = W.make_masked(3, 70, 144, 256, seed=83, masked_m=[0, 70, 33])
    dv = {k: to_dev(md[k]) for k in ("a", "b", "sb", "masked_m")}
    sa_cm = col_major(md["sa"], 70)                       # [3, 70, 2], leading dimension 72
    out, ref_out = sentinel_like((3, 70, 144)), sentinel_like((3, 70, 144))
    say("m_grouped_gemm_fp8_fp8_bf16_nt_masked")
    dg.m_grouped_gemm_fp8_fp8_bf16_nt_masked((dv["a"], sa_cm), (dv["b"], dv["sb"]), out, dv["masked_m"])
    dg.dg_m_grouped_gemm_fp8_masked(dv["a"], to_dev(md["sa"]), dv["b"], dv["sb"], ref_out, dv["masked_m"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref_out))


def test_num_sms_names():
    try:
        dg.set_num_sms(64)
        assert dg.get_num_sms() == 64
    finally:
        dg.set_num_sms(0)
