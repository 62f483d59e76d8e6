"""GPU parity of the FP8 cast kernels (the prior-kernel cast the README leaves to the
caller) against the oracle's quantiser: codes and scales must match bit for bit, for
E4M3 output and for E5M2 output (the blog's other FP8 format)."""
import numpy as np
import pytest

import fp8_block_scaled_e4m3_amd as dg
import workloads as W
from tests.gpu_support import bits, check_values, require_gpu, say, sentinel_like, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()
    dg.load_library()


def recipe(rows, k, block_rows, seed):
    rng = np.random.default_rng(seed)
    return W._scaled_normals(rng, rows, k, block_rows)


def specials(x):
    """Plant zeros, signed zeros, huge and tiny values, NaN and inf in known places."""
    x = x.copy()
    k = x.shape[1]
    x[0, :128] = 0.0                          # all-zero block -> scale 1
    x[1, :128] = -0.0
    x[1, 5] = 0.0
    x[2, :128] = np.float32(1e-30)            # subnormal-range codes after scaling
    x[2, 7] = np.float32(3.0)
    x[3, k - 2] = np.float32(1e30)            # one huge value: the rest round to 0 / tiny
    x[4, k // 2] = np.nan                     # NaN ignored by amax, coded 0x7F
    x[5, k - 1] = np.inf                      # amax inf: others -> +-0, inf -> NaN code
    x[6, :128] = np.float32(448.0) * np.linspace(-1, 1, 128, dtype=np.float32)
    x[7, :] = np.float32(2.0) ** ((np.arange(k) % 48) - 30).astype(np.float32)   # wide magnitude range
    if x.shape[0] > 8:
        x[8, :128] = np.float32(1e-40) * np.arange(-64, 64, dtype=np.float32)    # fp32-subnormal block: tiny scale
    return x


def as_bf16(x):
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t, t.to(torch.float32).numpy()


def gpu_1x128(x_t, rows, k, fmt="e4m3"):
    import torch
    q = torch.empty((rows, k), dtype=torch.uint8, device="cuda:0")
    sa = torch.full((k // 128, W.ld_sa_for(rows)), -1.0, device="cuda:0")
    if fmt == "e4m3":
        dg.dg_quantize_fp8_1x128(x_t, q, sa)
    else:
        dg.dg_quantize_fp8_1x128_fmt(x_t, q, sa, q_fmt=fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sa.cpu().numpy()


def gpu_128x128(x_t, rows, k, fmt="e4m3"):
    import torch
    q = torch.empty((rows, k), dtype=torch.uint8, device="cuda:0")
    sb = torch.full((-(-rows // 128), k // 128), -1.0, device="cuda:0")
    if fmt == "e4m3":
        dg.dg_quantize_fp8_128x128(x_t, q, sb)
    else:
        dg.dg_quantize_fp8_128x128_fmt(x_t, q, sb, q_fmt=fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sb.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


# K/128 = 1, 3, 5: a thread's blocks lie GPW blocks apart; 8, 12: runs of four
# consecutive K blocks per thread (33 x 12 blocks leaves a partial last workgroup)
@pytest.mark.parametrize("rows,k", [(1, 128), (7, 384), (300, 640), (129, 1024), (33, 1536)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_1x128_bit_exact(orc, rows, k, dtype, fmt):
    import torch
    x = recipe(rows, k, 1, seed=rows * 7 + k)
    if rows >= 8:
        x = specials(x)
    if dtype == "bf16":
        xt, x = as_bf16(x)
        xt = xt.to("cuda:0")
    else:
        xt = to_dev(x)
    say(f"quant 1x128 {rows}x{k} {dtype} {fmt}")
    q, sa = gpu_1x128(xt, rows, k, fmt)
    rq, rsa = orc.quantize_rows_1x128(x, fmt)
    assert np.array_equal(q, rq), f"{np.sum(q != rq)} codes differ"
    assert same_bits(sa[:, :rows], rsa)
    assert np.all(sa[:, rows:] == -1.0)                     # padding columns untouched


def e4m3_rounding_grid():
    """fp32 values at and around every E4M3 rounding decision in [-448, 448]: each
    representable value, each tie between neighbours and the fp32 values one ulp to
    either side of it, for normal and subnormal codes, plus values that round to 0."""
    vals = []
    for e in range(-9, 9):                       # E4M3 exponents (normal from -6, spacing 2^(e-3))
        for m in range(16):
            for frac in (0.0, 0.5):
                v = np.float32(2.0 ** e * (1 + (m + frac) / 8)) if e >= -6 else np.float32((m + frac) * 2.0 ** -9)
                vals += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1e9))]
    vals += [np.float32(2.0 ** -10), np.float32(2.0 ** -11), np.float32(1e-20), np.float32(0.0)]
    v = np.array(vals, np.float32)
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_quant_conversion_grid_bit_exact(orc):
    """With 448 in every block the scale is exactly 1, so the codes are the E4M3
    conversion itself: every rounding decision of the format, both signs, compared
    with the oracle's encoder."""
    grid = e4m3_rounding_grid()
    per = 127
    nblk = -(-grid.size // per)
    nblk += -nblk % 4                             # four blocks per row
    body = np.resize(grid, nblk * per).reshape(nblk, per)
    x = np.concatenate([np.full((nblk, 1), 448.0, np.float32), body], axis=1).reshape(-1, 128 * 4)
    rows = x.shape[0]
    q, sa = gpu_1x128(to_dev(x), rows, x.shape[1])
    rq, rsa = orc.quantize_rows_1x128(x)
    assert np.all(sa[:, :rows] == 1.0)
    assert np.array_equal(q, rq), f"{np.sum(q != rq)} codes differ"


def e5m2_rounding_grid():
    """fp32 values at and around every E5M2 rounding decision in [-57344, 57344]: each
    representable value, each tie between neighbours and the fp32 values one ulp to
    either side of it, for normal and subnormal codes, plus values that round to 0."""
    vals = []
    for e in range(-17, 16):                     # E5M2 exponents (normal from -14, spacing 2^(e-2))
        for m in range(8):
            for frac in (0.0, 0.5):
                v = np.float32(2.0 ** e * (1 + (m + frac) / 4)) if e >= -14 else np.float32((m + frac) * 2.0 ** -16)
                vals += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(1e9))]
    vals += [np.float32(2.0 ** -17), np.float32(2.0 ** -18), np.float32(1e-30), np.float32(0.0)]
    v = np.array(vals, np.float32)
    v = v[np.abs(v) <= 57344]
    return np.concatenate([v, -v])


def test_quant_e5m2_conversion_grid_bit_exact(orc):
    """With 57344 in every block the E5M2 scale is exactly 1, so the codes are the E5M2
    conversion itself: every rounding decision of the format, both signs, compared
    with the oracle's encoder."""
    grid = e5m2_rounding_grid()
    per = 127
    nblk = -(-grid.size // per)
    nblk += -nblk % 4                             # four blocks per row
    body = np.resize(grid, nblk * per).reshape(nblk, per)
    x = np.concatenate([np.full((nblk, 1), 57344.0, np.float32), body], axis=1).reshape(-1, 128 * 4)
    rows = x.shape[0]
    q, sa = gpu_1x128(to_dev(x), rows, x.shape[1], "e5m2")
    rq, rsa = orc.quantize_rows_1x128(x, "e5m2")
    assert np.all(sa[:, :rows] == 1.0)
    assert np.array_equal(q, rq), f"{np.sum(q != rq)} codes differ"


@pytest.mark.parametrize("rows,k", [(128, 128), (200, 384), (1, 256), (385, 512)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_128x128_bit_exact(orc, rows, k, dtype, fmt):
    x = recipe(rows, k, 128, seed=rows * 11 + k)
    if rows >= 8:
        x = specials(x)
    if dtype == "bf16":
        xt, x = as_bf16(x)
        xt = xt.to("cuda:0")
    else:
        xt = to_dev(x)
    say(f"quant 128x128 {rows}x{k} {dtype} {fmt}")
    q, sb = gpu_128x128(xt, rows, k, fmt)
    rq, rsb = orc.quantize_blocks_128x128(x, fmt)
    assert np.array_equal(q, rq), f"{np.sum(q != rq)} codes differ"
    assert same_bits(sb, rsb)


def test_quant_full_size_prefill_operands(orc):
    """The prefill workload's A (4096x7168) and B (7168x7168) cast on the GPU equal the
    oracle's cast and the shared generator's (torch-based) cast."""
    rng = np.random.default_rng(0)
    xa = W._scaled_normals(rng, 4096, 7168, 1)
    say("quant 1x128 4096x7168 f32")
    q, sa = gpu_1x128(to_dev(xa), 4096, 7168)
    rq, rsa = orc.quantize_rows_1x128(xa)
    assert np.array_equal(q, rq) and same_bits(sa, rsa)
    gq, gsa = W.quant_rows_1x128(xa)
    assert np.array_equal(q, gq) and same_bits(sa, gsa)
    del xa
    xb = W._scaled_normals(rng, 7168, 7168, 128)
    say("quant 128x128 7168x7168 f32")
    q, sb = gpu_128x128(to_dev(xb), 7168, 7168)
    rq, rsb = orc.quantize_blocks_128x128(xb)
    assert np.array_equal(q, rq) and same_bits(sb, rsb)


def test_cast_then_gemm_end_to_end(orc):
    """GPU cast of fp32 operands followed by the GPU GEMM matches the oracle GEMM of the
    oracle's cast of the same operands."""
    import torch
    m, n, k = 320, 272, 640
    rng = np.random.default_rng(5)
    xa, xb = W._scaled_normals(rng, m, k, 1), W._scaled_normals(rng, n, k, 128)
    qa = torch.empty((m, k), dtype=torch.uint8, device="cuda:0")
    sa = torch.empty((k // 128, W.ld_sa_for(m)), device="cuda:0")
    qb = torch.empty((n, k), dtype=torch.uint8, device="cuda:0")
    sb = torch.empty((-(-n // 128), k // 128), device="cuda:0")
    d = sentinel_like((m, n))
    dg.dg_quantize_fp8_1x128(to_dev(xa), qa, sa)
    dg.dg_quantize_fp8_128x128(to_dev(xb), qb, sb)
    dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d)
    torch.cuda.synchronize()
    ra, rsa = orc.quantize_rows_1x128(xa)
    rb, rsb = orc.quantize_blocks_128x128(xb)
    check_values(bits(d), orc.gemm_fp8_nt(ra, rsa, rb, rsb), "cast + gemm")


def test_e5m2_cast_then_gemm_end_to_end(orc):
    """E5M2 casts on the GPU (selected by float8_e5m2 output tensors) followed by the GPU
    GEMM with E5M2 operands match the oracle GEMM of the oracle's E5M2 casts."""
    import torch
    m, n, k = 192, 208, 512
    rng = np.random.default_rng(6)
    xa, xb = W._scaled_normals(rng, m, k, 1), W._scaled_normals(rng, n, k, 128)
    qa = torch.empty((m, k), dtype=torch.float8_e5m2, device="cuda:0")
    sa = torch.empty((k // 128, W.ld_sa_for(m)), device="cuda:0")
    qb = torch.empty((n, k), dtype=torch.float8_e5m2, device="cuda:0")
    sb = torch.empty((-(-n // 128), k // 128), device="cuda:0")
    d = sentinel_like((m, n))
    dg.dg_quantize_fp8_1x128(to_dev(xa), qa, sa)
    dg.dg_quantize_fp8_128x128(to_dev(xb), qb, sb)
    dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d)
    torch.cuda.synchronize()
    ra, rsa = orc.quantize_rows_1x128(xa, "e5m2")
    rb, rsb = orc.quantize_blocks_128x128(xb, "e5m2")
    assert np.array_equal(qa.view(torch.uint8).cpu().numpy(), ra)
    assert np.array_equal(qb.view(torch.uint8).cpu().numpy(), rb)
    check_values(bits(d), orc.gemm_fp8_nt(ra, rsa, rb, rsb, a_fmt="e5m2", b_fmt="e5m2"), "e5m2 cast + gemm")


def test_quant_validation_errors():
    import torch
    x = torch.zeros((4, 200), device="cuda:0")
    q = torch.zeros((4, 200), dtype=torch.uint8, device="cuda:0")
    sa = torch.zeros((2, 4), device="cuda:0")
    with pytest.raises(dg.DGError) as e:
        dg.dg_quantize_fp8_1x128(x, q, sa)
    assert e.value.status == dg.DG_ERR_UNSUPPORTED
    x = torch.zeros((4, 256), device="cuda:0")
    q = torch.zeros((4, 256), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(ValueError):
        dg.dg_quantize_fp8_1x128_fmt(x, q, sa, q_fmt="e3m4")


def tie_panel(fmt, scale_exps, seed):
    """128-row panels, one per scale s: every 1x128 block is [FMAX*s, then values p and
    their fp32 neighbours, p = t*s for the format's values and rounding ties t], so that
    each 1x128 and each 128x128 block gets the scale s exactly and its quotients land on
    and beside every rounding decision.  The scales have 18-bit significands and the t
    at most 5, so every p is exact."""
    rng = np.random.default_rng(seed)
    fmax = 448.0 if fmt == "e4m3" else 57344.0
    ties = []
    if fmt == "e4m3":
        for e in range(-9, 9):
            for m in range(16):
                for frac in (0.0, 0.5):
                    ties.append(2.0 ** e * (1 + (m + frac) / 8) if e >= -6 else (m + frac) * 2.0 ** -9)
    else:
        for e in range(-17, 16):
            for m in range(8):
                for frac in (0.0, 0.5):
                    ties.append(2.0 ** e * (1 + (m + frac) / 4) if e >= -14 else (m + frac) * 2.0 ** -16)
    t = np.array(sorted(set(ties)), np.float64)
    t = t[t <= fmax]
    t = np.concatenate([t, -t])
    panels = []
    for e in scale_exps:
        s = (1.0 + int(rng.integers(0, 1 << 17)) / 2.0 ** 17) * 2.0 ** e
        p = t * s
        p32 = p.astype(np.float32)
        assert np.all(p32.astype(np.float64) == p)                              # exact products
        vals = np.stack([p32, np.nextafter(p32, np.float32(-np.inf)), np.nextafter(p32, np.float32(np.inf))], 1)
        flat = vals.reshape(-1)
        step = -(-flat.size // 128)                     # the 128 rows together cover every value
        x = np.empty((128, 4 * 128), np.float32)
        for r in range(128):
            row = np.resize(np.roll(flat, -step * r), 4 * 127).reshape(4, 127)
            x[r] = np.concatenate([np.full((4, 1), np.float32(fmax * s)), row], axis=1).reshape(-1)
        panels.append(x)
    return np.concatenate(panels)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quant_tiny_and_boundary_scales_bit_exact(orc, fmt):
    """Blocks whose scales sit far below the fast path (2^-120, 2^-100, 2^-80: the
    software path), at its lower edge (2^-65, 2^-64, 2^-63) and in the normal range,
    each with values on and beside every rounding decision: codes and scales of both
    casts equal the oracle's bit for bit."""
    exps = [-120, -100, -80, -65, -64, -63, -40, 0, 30] if fmt == "e4m3" else [-110, -90, -65, -64, -63, 0, 20]
    x = tie_panel(fmt, exps, seed=17 if fmt == "e4m3" else 18)
    rows, k = x.shape
    say(f"quant tiny/boundary scales {fmt}: {rows}x{k}")
    q, sa = gpu_1x128(to_dev(x), rows, k, fmt)
    rq, rsa = orc.quantize_rows_1x128(x, fmt)
    assert np.array_equal(q, rq), f"1x128: {np.sum(q != rq)} codes differ"
    assert same_bits(sa[:, :rows], rsa)
    q, sb = gpu_128x128(to_dev(x), rows, k, fmt)
    rq, rsb = orc.quantize_blocks_128x128(x, fmt)
    assert np.array_equal(q, rq), f"128x128: {np.sum(q != rq)} codes differ"
    assert same_bits(sb, rsb)


@pytest.mark.parametrize("rows,kb,groups", [(1, 1, 1), (37, 5, 1), (300, 56, 1), (4097, 16, 1), (70, 9, 3)])
def test_transform_sa_mn_major(rows, kb, groups):
    """Row-major per-row scales to the GEMMs' MN-major layout with an aligned leading
    dimension: a plain transpose, bit for bit; padding columns untouched."""
    import torch
    rng = np.random.default_rng(rows + kb)
    src = rng.standard_normal((groups, rows, kb + 3)).astype(np.float32)   # ld_in = kb + 3
    x = to_dev(src)[:, :, :kb]
    ld = dg.dg_get_aligned_ld_sa(rows)
    out = torch.full((groups, kb, ld), 7.0, device="cuda:0")
    say(f"transform sa rows={rows} kb={kb} groups={groups}")
    dg.dg_transform_sa_mn_major(x if groups > 1 else x[0], out if groups > 1 else out[0])
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert same_bits(got[:, :, :rows], np.ascontiguousarray(src[:, :, :kb].transpose(0, 2, 1)))
    assert np.all(got[:, :, rows:] == 7.0)


def test_transformed_sa_feeds_the_gemm(orc):
    """The cast's row-major scales (as the pages' callers hold them) transformed on the GPU
    and used by the dense GEMM give the oracle's result."""
    import torch
    dd = W.make_dense(200, 256, 512, seed=61)
    rowmajor = to_dev(np.ascontiguousarray(dd["sa"][:, :200].T))           # [rows, K/128]
    sa = dg.dg_transform_sa_mn_major(rowmajor)
    d = sentinel_like((200, 256))
    dg.dg_gemm_fp8_nt(to_dev(dd["a"]), sa, to_dev(dd["b"]), to_dev(dd["sb"]), d)
    torch.cuda.synchronize()
    check_values(bits(d), orc.gemm_fp8_nt(dd["a"], dd["sa"], dd["b"], dd["sb"]), "transformed sa + gemm")
