"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties one part of the oracle to a closed form, a value the pages print,
an independent library routine, exact rational brute force or an invariant of
the mathematics, so that a plausible slip (a wrong bias, a dropped sign, a
transposed operand, a wrong scale index, a double rounding) fails here.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_e4m3_values():
    """float64 value of every E4M3FN byte, decoded by torch (independent of the oracle)."""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def bf16_bits_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


# --------------------------------------------------------------------------- E4M3 decode
def test_e4m3_golden_max(orc):
    dec = orc.e4m3_decode_table()
    for line in open(os.path.join(GOLDEN, "e4m3_max.txt")):
        if line.startswith("#") or not line.strip():
            continue
        byte, val = line.split()
        assert dec[int(byte, 16)] == float(val)
    finite = dec[np.isfinite(dec)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_e4m3_table_closed_forms(orc):
    dec = orc.e4m3_decode_table()
    nan = np.isnan(dec)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert not np.isinf(dec).any()
    assert dec[0x38] == 1.0                       # s=0 e=7 f=0
    assert dec[0x08] == 2.0 ** -6                 # smallest normal
    assert dec[0x01] == 2.0 ** -9                 # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert dec[0x00] == 0.0 and math.copysign(1.0, dec[0x80]) == -1.0
    for b in range(0x7F):
        assert dec[b | 0x80] == -dec[b]
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)               # strictly increasing codes
    units = dec[~nan] * 512.0                     # every value is an integer * 2^-9
    assert np.all(units == np.round(units)) and np.abs(units).max() == 229376


def test_e4m3_table_matches_torch(orc):
    assert np.array_equal(orc.e4m3_decode_table(), torch_e4m3_values(), equal_nan=True)


# --------------------------------------------------------------------------- E4M3 encode
@pytest.mark.parametrize("x,byte", [
    (1.0 + 2.0 ** -4, 0x38),       # tie between 1.0 and 1.125 -> even mantissa 1.0
    (1.0 + 3 * 2.0 ** -4, 0x3A),   # tie between 1.125 and 1.25 -> 1.25
    (1.0 + 2.0 ** -4 + 2.0 ** -20, 0x39),
    (2.0 ** -10, 0x00),            # half the smallest subnormal -> 0 (even)
    (3 * 2.0 ** -10, 0x02),        # tie between 2^-9 and 2^-8 -> 2^-8
    (460.0, 0x7E),                 # saturates at 448
    (1e30, 0x7E),
    (-460.0, 0xFE),
    (-0.0, 0x80),
    (0.0, 0x00),
    (float("nan"), 0x7F),
    (15 * 2.0 ** -10, 0x08),       # 7.5 * 2^-9 rounds up into the smallest normal
])
def test_e4m3_encode_closed_forms(orc, x, byte):
    assert orc.e4m3_encode(x) == byte


def test_e4m3_encode_roundtrip_and_torch(orc):
    dec = orc.e4m3_decode_table()
    for b in range(256):
        if b in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(dec[b]) == b
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(3000) * 50,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),          # subnormal range
        (np.arange(-448 * 512, 448 * 512 + 1, 37) / 512.0),  # many exact ties
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_quantisers_match_generator(orc):
    """The oracle's quantiser and the shared generator's torch-based cast agree bit for bit."""
    x = np.random.default_rng(3).standard_normal((261, 700)).astype(np.float32)
    x[5, :128] = 0.0                                        # amax == 0 block -> scale 1
    q1, s1 = W.quant_rows_1x128(x)
    qa, s2 = orc.quantize_rows_1x128(x)
    assert np.array_equal(q1, qa) and np.array_equal(s1[:, :261], s2)
    q1, s1 = W.quant_blocks_128x128(x)
    q2, s2 = orc.quantize_blocks_128x128(x)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    dec = orc.e4m3_decode_table()
    # every non-zero 1x128 block reaches exactly +-448 at its amax element
    blk = np.abs(dec[qa[:, :640]].reshape(261, 5, 128)).max(axis=2)
    assert np.all((blk == 448.0) | (blk == 0.0)) and (blk == 0.0).sum() == 1
    # every non-zero 128x128 block of the B-side cast reaches +-448 somewhere
    blk = np.abs(dec[q2[:256, :640]].reshape(2, 128, 5, 128)).max(axis=(1, 3))
    assert np.all(blk == 448.0)


# --------------------------------------------------------------------------- BF16
@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),             # tie -> even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),         # tie -> even (1 + 2^-6)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie: single rounding from double
    (-2.0, 0xC000),
    (2.0 ** -133, 0x0001),                 # smallest subnormal
    (2.0 ** -134, 0x0000),                 # half of it -> 0 (even)
    (3 * 2.0 ** -134, 0x0002),
    (2.0 ** -126, 0x0080),                 # smallest normal
    (2.0 ** 128, 0x7F80),                  # overflow -> inf
    (-(2.0 ** 127) * (2 - 2.0 ** -8), 0xFF80),  # rounds past the largest finite -> -inf
    ((2.0 ** 127) * (2 - 2.0 ** -7), 0x7F7F),   # largest finite
    (float("nan"), 0x7FC0),
    (-0.0, 0x8000),
])
def test_bf16_closed_forms(orc, x, bits):
    assert orc.bf16_encode(x) == bits


def test_bf16_matches_torch_on_floats(orc):
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000),
                        rng.standard_normal(500) * 1e-39]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_encode(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------- exact block sums
def test_block_dot_all_byte_pairs(orc):
    vals = torch_e4m3_values()
    finite = [b for b in range(256) if b not in (0x7F, 0xFF)]
    for a in finite[::3]:
        for b in finite:
            assert orc.block_dot([a], [b]) == vals[a] * vals[b]


def test_block_dot_equals_int64_sum(orc):
    vals = torch_e4m3_values()
    units = np.where(np.isnan(vals), 0, vals * 512).astype(np.int64)
    rng = np.random.default_rng(5)
    for trial in range(200):
        a = rng.integers(0, 256, 128).astype(np.uint8)
        b = rng.integers(0, 256, 128).astype(np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x7E
        b[(b & 0x7F) == 0x7F] = 0xFE
        exact = int((units[a] * units[b]).sum())
        got = orc.block_dot(a, b)
        assert got * 2 ** 18 == exact
        perm = rng.permutation(128)
        assert orc.block_dot(a[perm], b[perm]) == got       # order never matters


# --------------------------------------------------------------------------- E5M2 (second operand format)
def torch_e5m2_values():
    """float64 value of every E5M2 byte, decoded by torch (independent of the oracle)."""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e5m2) \
        .to(torch.float64).numpy()


def test_e5m2_table_closed_forms(orc):
    dec = orc.e5m2_decode_table()
    assert dec[0x00] == 0.0 and math.copysign(1.0, dec[0x80]) == -1.0
    assert dec[0x01] == 2.0 ** -16 and dec[0x03] == 3 * 2.0 ** -16       # subnormals
    assert dec[0x04] == 2.0 ** -14                                          # smallest normal
    assert dec[0x3C] == 1.0 and dec[0x3D] == 1.25 and dec[0x40] == 2.0
    assert dec[0x7B] == 57344.0                                             # largest finite
    assert dec[0x7C] == math.inf and dec[0xFC] == -math.inf
    assert all(math.isnan(dec[b]) for b in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    for b in range(0x7C):
        assert dec[b | 0x80] == -dec[b] or (b == 0 and dec[0x80] == 0.0)
        if b:
            assert dec[b] > dec[b - 1]


def test_e5m2_table_matches_torch(orc):
    dec, ref = orc.e5m2_decode_table(), torch_e5m2_values()
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(dec[ok], ref[ok])


# --------------------------------------------------------------------------- E5M2 encode
@pytest.mark.parametrize("x,byte", [
    (1.0, 0x3C),
    (1.125, 0x3C),                 # tie between 1.0 and 1.25 -> even mantissa 1.0
    (1.375, 0x3E),                 # tie between 1.25 and 1.5 -> 1.5
    (1.125 + 2.0 ** -20, 0x3D),
    (2.0 ** -16, 0x01),            # smallest subnormal
    (2.0 ** -17, 0x00),            # half of it -> 0 (even)
    (3 * 2.0 ** -17, 0x02),        # tie between 2^-16 and 2^-15 -> 2^-15
    (7 * 2.0 ** -17, 0x04),        # 3.5 * 2^-16 rounds up into the smallest normal 2^-14
    (57344.0, 0x7B),               # largest finite
    (60000.0, 0x7B),               # saturates at 57344
    (1e30, 0x7B),
    (float("inf"), 0x7B),
    (-60000.0, 0xFB),
    (-0.0, 0x80),
    (0.0, 0x00),
    (float("nan"), 0x7F),
])
def test_e5m2_encode_closed_forms(orc, x, byte):
    assert orc.e5m2_encode(x) == byte


def test_e5m2_encode_roundtrip_and_torch(orc):
    """Every finite byte encodes back to itself; on finite values within the range,
    including every midpoint between neighbouring E5M2 values and the fp32 values
    next to it, the encoder equals torch's float32 -> float8_e5m2 cast."""
    dec = torch_e5m2_values()
    fin = [b for b in range(256) if np.isfinite(dec[b])]
    for b in fin:
        assert orc.e5m2_encode(dec[b]) == b
    pos = np.unique(np.abs(dec[fin]))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    rng = np.random.default_rng(9)
    vals = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        rng.standard_normal(3000).astype(np.float32) * 5000,
        rng.uniform(-2.0 ** -13, 2.0 ** -13, 2000).astype(np.float32),   # subnormal range
    ]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    vals = vals[np.abs(vals) <= 57344.0]
    ref = torch.from_numpy(vals).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = np.array([orc.e5m2_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_e5m2_quantisers_match_generator(orc):
    """E5M2 casts: the oracle's quantiser and the generator's torch-based cast agree bit
    for bit, and every non-zero block reaches +-57344 at its amax."""
    x = np.random.default_rng(4).standard_normal((261, 700)).astype(np.float32)
    x[7, 128:256] = 0.0
    q1, s1 = W.quant_rows_1x128(x, "e5m2")
    qa, s2 = orc.quantize_rows_1x128(x, "e5m2")
    assert np.array_equal(q1, qa) and np.array_equal(s1[:, :261], s2)
    q1, s1 = W.quant_blocks_128x128(x, "e5m2")
    q2, s2 = orc.quantize_blocks_128x128(x, "e5m2")
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    dec = orc.e5m2_decode_table()
    blk = np.abs(dec[qa[:, :640]].reshape(261, 5, 128)).max(axis=2)
    assert np.all((blk == 57344.0) | (blk == 0.0)) and (blk == 0.0).sum() == 1
    blk = np.abs(dec[q2[:256, :640]].reshape(2, 128, 5, 128)).max(axis=(1, 3))
    assert np.all(blk == 57344.0)
    # the same bytes through the format path equal the plain path for E4M3
    assert np.array_equal(orc.quantize_rows_1x128(x, "e4m3")[0], orc.quantize_rows_1x128(x)[0])


@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e4m3")])
def test_block_dot_fmt_is_exact_sum_rounded_once(orc, fa, fb):
    """The block sum with E5M2 operands needs up to ~70 bits: it must equal the exact
    rational sum rounded once to fp64 (Python's Fraction -> float rounds correctly),
    also for blocks of the largest values where an fp64 running sum would round."""
    va = torch_e5m2_values() if fa == "e5m2" else torch_e4m3_values()
    vb = torch_e5m2_values() if fb == "e5m2" else torch_e4m3_values()
    fin_a = np.array([b for b in range(256) if np.isfinite(va[b])], np.uint8)
    fin_b = np.array([b for b in range(256) if np.isfinite(vb[b])], np.uint8)
    rng = np.random.default_rng(6)
    for trial in range(150):
        a, b = rng.choice(fin_a, 128), rng.choice(fin_b, 128)
        if trial % 3 == 0:                          # extremes: the largest and smallest magnitudes
            a[::2] = fin_a[np.argmax(np.abs(va[fin_a]))]
            b[1::2] = fin_b[np.argmin(np.where(vb[fin_b] == 0, np.inf, np.abs(vb[fin_b])))]
        exact = sum(Fraction(float(va[x])) * Fraction(float(vb[y])) for x, y in zip(a, b))
        assert orc.block_dot_fmt(a, b, fa, fb) == float(exact)
        if fa == fb == "e4m3":
            assert orc.block_dot_fmt(a, b) == orc.block_dot(a, b)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_gemm_fmt_equals_exact_rational(orc, fa, fb):
    """The dense GEMM with E5M2 operands against exact rational brute force rounded once
    to BF16 (several K blocks, a short last block, two B-scale blocks)."""
    m, n, k = 3, 133, 300
    rng = np.random.default_rng(7 + len(fa + fb))
    va = torch_e5m2_values() if fa == "e5m2" else torch_e4m3_values()
    vb = torch_e5m2_values() if fb == "e5m2" else torch_e4m3_values()
    fin_a = np.array([b for b in range(256) if np.isfinite(va[b])], np.uint8)
    fin_b = np.array([b for b in range(256) if np.isfinite(vb[b])], np.uint8)
    a, b = rng.choice(fin_a, (m, k)), rng.choice(fin_b, (n, k))
    kb, nb = -(-k // 128), -(-n // 128)
    sa = (rng.uniform(0.5, 2, (kb, m)) * 2.0 ** rng.integers(-12, 0, (kb, m))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, (nb, kb)) * 2.0 ** rng.integers(-12, 0, (nb, kb))).astype(np.float32)
    d = orc.gemm_fp8_nt(a, sa, b, sb, a_fmt=fa, b_fmt=fb)
    for i in range(m):
        for j in range(0, n, 7):
            tot = Fraction(0)
            for blk in range(kb):
                ks = range(blk * 128, min(k, blk * 128 + 128))
                p = sum(Fraction(float(va[a[i, t]])) * Fraction(float(vb[b[j, t]])) for t in ks)
                tot += Fraction(float(sa[blk, i])) * Fraction(float(sb[j // 128, blk])) * p
            assert d[i, j] == _exact_bf16(tot), (i, j)


def test_gemm_fmt_e4m3_matches_plain_path(orc):
    rng = np.random.default_rng(8)
    a, b = _rand_fp8(rng, (5, 256)), _rand_fp8(rng, (40, 256))
    sa = rng.uniform(0.5, 2, (2, 8)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (1, 2)).astype(np.float32)
    plain = orc.gemm_fp8_nt(a, sa, b, sb)
    lib = orc._load()
    d = np.zeros((5, 40), np.uint16)
    lib.orc_gemm_fp8_nt_fmt(orc._ptr(a), 256, orc._ptr(sa), 8, orc._ptr(b), 256, orc._ptr(sb),
                            orc._ptr(d), 40, None, 5, 40, 256, 0, 0, 1)
    assert np.array_equal(d, plain)


# --------------------------------------------------------------------------- whole GEMM
def _exact_bf16(x: Fraction) -> int:
    """Round an exact rational to BF16 (RNE), written with rationals only."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    r = a / q
    n = r.numerator // r.denominator
    frac = r - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n < 128:
        return sign | n
    if n == 256:
        n, e = 128, e + 1
    assert e <= 127
    return sign | ((e + 127) << 7) | (n - 128)


def _rand_fp8(rng, shape):
    x = rng.integers(0, 256, shape).astype(np.uint8)
    x[(x & 0x7F) == 0x7F] = 0x3C
    return x


@pytest.mark.parametrize("m,n,k", [(2, 3, 384), (3, 133, 300), (1, 257, 128)])
def test_gemm_equals_exact_rational(orc, m, n, k):
    """Brute force in exact rationals, rounded once to BF16: covers several K blocks, a
    short last K block and columns that use different 128-row B-scale blocks."""
    rng = np.random.default_rng(m * 1000 + n + k)
    a, b = _rand_fp8(rng, (m, k)), _rand_fp8(rng, (n, k))
    kb, nb = -(-k // 128), -(-n // 128)
    sa = (rng.uniform(0.5, 2, (kb, m)) * 2.0 ** rng.integers(-6, 6, (kb, m))).astype(np.float32)
    sb = (rng.uniform(0.5, 2, (nb, kb)) * 2.0 ** rng.integers(-6, 6, (nb, kb))).astype(np.float32)
    vals = torch_e4m3_values()
    fa = [[Fraction(float(vals[x])) for x in row] for row in a]
    fb = [[Fraction(float(vals[x])) for x in row] for row in b]
    d, acc = orc.gemm_fp8_nt(a, sa, b, sb, want_acc=True)
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            for blk in range(kb):
                p = sum(fa[i][t] * fb[j][t] for t in range(blk * 128, min(k, blk * 128 + 128)))
                tot += Fraction(float(sa[blk, i])) * Fraction(float(sb[j // 128, blk])) * p
            assert d[i, j] == _exact_bf16(tot), (i, j)
            assert abs(Fraction(acc[i, j]) - tot) <= abs(tot) * Fraction(1, 2 ** 49) + Fraction(1, 2 ** 200)


def test_gemm_one_hot(orc):
    rng = np.random.default_rng(1)
    m, n, k = 64, 160, 512
    vals = torch_e4m3_values()
    for trial in range(10):
        a = np.zeros((m, k), np.uint8)
        b = np.zeros((n, k), np.uint8)
        i, j, t = rng.integers(m), rng.integers(n), rng.integers(k)
        a[i, t], b[j, t] = rng.integers(1, 0x7E), rng.integers(0x81, 0xFE)
        sa = rng.uniform(0.1, 3, (k // 128, m)).astype(np.float32)
        sb = rng.uniform(0.1, 3, (2, k // 128)).astype(np.float32)
        d = orc.gemm_fp8_nt(a, sa, b, sb)
        expect = float(sa[t // 128, i]) * float(sb[j // 128, t // 128]) * vals[a[i, t]] * vals[b[j, t]]
        assert d[i, j] == _exact_bf16(Fraction(expect))
        d[i, j] = 0
        assert not d.any()


def test_gemm_identity_returns_scaled_transpose(orc):
    rng = np.random.default_rng(2)
    a = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(a, 0x38)                      # 1.0
    b = _rand_fp8(rng, (128, 128))
    sa = np.ones((1, 128), np.float32)
    sb = np.array([[0.75]], np.float32)
    d = orc.gemm_fp8_nt(a, sa, b, sb)
    vals = torch_e4m3_values()
    expect = 0.75 * vals[b.T]                      # D[m, n] = sB * dec(B[n, m])
    ref = torch.from_numpy(expect.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = np.where(ref == 0x8000, 0, ref)          # an exact zero sum is +0 in the oracle
    assert np.array_equal(d, ref)


def test_gemm_unit_scales_is_textbook_matmul(orc):
    """With all scales 1 and K = 128 the fp64 accumulator is the plain product of the
    decoded matrices, which numpy computes exactly here (all sums fit 53 bits)."""
    rng = np.random.default_rng(4)
    a, b = _rand_fp8(rng, (70, 128)), _rand_fp8(rng, (90, 128))
    vals = torch_e4m3_values()
    _, acc = orc.gemm_fp8_nt(a, np.ones((1, 70), np.float32), b, np.ones((1, 1), np.float32),
                             want_acc=True)
    assert np.array_equal(acc, vals[a] @ vals[b].T)


def test_gemm_power_of_two_scale_invariance(orc):
    d0 = W.make_dense(96, 200, 384, seed=9)
    base = orc.gemm_fp8_nt(d0["a"], d0["sa"], d0["b"], d0["sb"])
    sa = d0["sa"].copy()
    sa[:, 17] *= 2.0 ** 5
    sa[:, 40] *= 2.0 ** -3
    out = orc.gemm_fp8_nt(d0["a"], sa, d0["b"], d0["sb"])
    f0, f1 = bf16_bits_to_f64(base), bf16_bits_to_f64(out)
    assert np.array_equal(f1[17], f0[17] * 32) and np.array_equal(f1[40], f0[40] / 8)
    mask = np.ones(96, bool)
    mask[[17, 40]] = False
    assert np.array_equal(out[mask], base[mask])
    sb = d0["sb"].copy()
    sb[1, :] *= 4.0                                 # second 128-column block of B only
    out = orc.gemm_fp8_nt(d0["a"], d0["sa"], d0["b"], sb)
    f1 = bf16_bits_to_f64(out)
    assert np.array_equal(f1[:, 128:], f0[:, 128:] * 4) and np.array_equal(out[:, :128], base[:, :128])


def test_gemm_zero_scale_equals_zeroed_block(orc):
    """Zeroing sA for one K block equals zeroing that block of A: the scale of block kb
    multiplies exactly the K columns of block kb."""
    d0 = W.make_dense(64, 130, 512, seed=10)
    sa = d0["sa"].copy()
    sa[2, :] = 0.0
    a = d0["a"].copy()
    a[:, 256:384] = 0
    assert np.array_equal(orc.gemm_fp8_nt(d0["a"], sa, d0["b"], d0["sb"]),
                          orc.gemm_fp8_nt(a, d0["sa"], d0["b"], d0["sb"]))


# --------------------------------------------------------------------------- grouped layouts
def test_contiguous_equals_dense_per_group(orc):
    counts = [130, 0, 1, 257]
    dd = W.make_contiguous(counts, n=144, k=256, seed=12)
    sentinel = np.full((dd["m_total"], 144), W.SENTINEL_BF16, np.uint16)
    out = orc.m_grouped_contiguous(dd["a"], dd["sa"], dd["b"], dd["sb"], dd["m_indices"], d_init=sentinel)
    off = 0
    for g, (c, p) in enumerate(zip(counts, W.padded(counts))):
        rows = slice(off, off + c)
        ref = orc.gemm_fp8_nt(dd["a"][rows], dd["sa"][:, off:off + c], dd["b"][g], dd["sb"][g])
        assert np.array_equal(out[rows], ref)
        assert np.all(out[off + c:off + p] == W.SENTINEL_BF16)
        off += p


def test_masked_equals_dense_and_keeps_sentinel(orc):
    mm = [0, 1, 17, 64, 70]
    dd = W.make_masked(5, 70, 144, 256, seed=13, masked_m=mm)
    sentinel = np.full((5, 70, 144), W.SENTINEL_BF16, np.uint16)
    out = orc.m_grouped_masked(dd["a"], dd["sa"], dd["b"], dd["sb"], dd["masked_m"], d_init=sentinel)
    for g, c in enumerate(mm):
        if c:
            ref = orc.gemm_fp8_nt(dd["a"][g, :c], dd["sa"][g][:, :c], dd["b"][g], dd["sb"][g])
            assert np.array_equal(out[g, :c], ref)
        assert np.all(out[g, c:] == W.SENTINEL_BF16)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")])
def test_grouped_fmt_equal_dense_fmt_per_group(orc, fa, fb):
    """With E5M2 operands the grouped layouts still equal the dense GEMM (pinned against
    exact rationals for every format pair) group by group, padding and masked rows
    untouched."""
    counts = [130, 0, 3]
    cd = W.make_contiguous(counts, n=144, k=256, seed=21, a_fmt=fa, b_fmt=fb)
    sentinel = np.full((cd["m_total"], 144), W.SENTINEL_BF16, np.uint16)
    out = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"], d_init=sentinel,
                                   a_fmt=fa, b_fmt=fb)
    off = 0
    for g, (c, p) in enumerate(zip(counts, W.padded(counts))):
        if c:
            ref = orc.gemm_fp8_nt(cd["a"][off:off + c], cd["sa"][:, off:off + c], cd["b"][g], cd["sb"][g],
                                  a_fmt=fa, b_fmt=fb)
            assert np.array_equal(out[off:off + c], ref)
        assert np.all(out[off + c:off + p] == W.SENTINEL_BF16)
        off += p
    mm = [0, 5, 40]
    md = W.make_masked(3, 40, 144, 256, seed=22, masked_m=mm, a_fmt=fa, b_fmt=fb)
    sentinel = np.full((3, 40, 144), W.SENTINEL_BF16, np.uint16)
    out = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], md["masked_m"], d_init=sentinel,
                               a_fmt=fa, b_fmt=fb)
    for g, c in enumerate(mm):
        if c:
            ref = orc.gemm_fp8_nt(md["a"][g, :c], md["sa"][g][:, :c], md["b"][g], md["sb"][g], a_fmt=fa, b_fmt=fb)
            assert np.array_equal(out[g, :c], ref)
        assert np.all(out[g, c:] == W.SENTINEL_BF16)


def test_grouped_fmt_e4m3_matches_plain_path(orc):
    counts = [70, 2]
    cd = W.make_contiguous(counts, n=48, k=256, seed=23)
    plain = orc.m_grouped_contiguous(cd["a"], cd["sa"], cd["b"], cd["sb"], cd["m_indices"])
    lib = orc._load()
    d = np.zeros_like(plain)
    lib.orc_m_grouped_contiguous_fmt(orc._ptr(cd["a"]), orc._ptr(cd["sa"]), cd["sa"].shape[1], orc._ptr(cd["b"]),
                                     orc._ptr(cd["sb"]), orc._ptr(d), None, orc._ptr(cd["m_indices"]),
                                     cd["m_total"], 48, 256, 2, 0, 0, 1)
    assert np.array_equal(d, plain)
    md = W.make_masked(2, 24, 48, 256, seed=24, masked_m=[24, 3])
    plain = orc.m_grouped_masked(md["a"], md["sa"], md["b"], md["sb"], md["masked_m"])
    d = np.zeros_like(plain)
    lib.orc_m_grouped_masked_fmt(orc._ptr(md["a"]), orc._ptr(md["sa"]), md["sa"].shape[2], orc._ptr(md["b"]),
                                 orc._ptr(md["sb"]), orc._ptr(d), None, orc._ptr(md["masked_m"]),
                                 2, 24, 48, 256, 0, 0, 1)
    assert np.array_equal(d, plain)


def test_masked_clamps_out_of_range_counts(orc):
    dd = W.make_masked(2, 16, 32, 128, seed=14, masked_m=[-5, 99])
    sentinel = np.full((2, 16, 32), W.SENTINEL_BF16, np.uint16)
    out = orc.m_grouped_masked(dd["a"], dd["sa"], dd["b"], dd["sb"], dd["masked_m"], d_init=sentinel)
    assert np.all(out[0] == W.SENTINEL_BF16) and not np.any(out[1] == W.SENTINEL_BF16)


# --------------------------------------------------------------------------- generator recipe
def test_zipf_split():
    c = W.zipf_counts(32768, 8, 1.1)
    assert sum(c) == 32768 and c == sorted(c, reverse=True)
    assert c == [13047, 6087, 3897, 2839, 2221, 1818, 1534, 1325]
    assert sum(W.padded(c)) == 33280


def test_generator_is_seeded_and_in_range():
    d1 = W.make_dense(128, 128, 512, seed=0)
    d2 = W.make_dense(128, 128, 512, seed=0)
    for key in ("a", "sa", "b", "sb"):
        assert np.array_equal(d1[key], d2[key])
    assert not np.any((d1["a"] & 0x7F) == 0x7F) and not np.any((d1["b"] & 0x7F) == 0x7F)
    # scales are amax/448 of N(0,1) data times 2^U(-4,4): within [2^-4 * 0.5/448, 2^4 * 6/448]
    assert d1["sa"][:, :128].min() > 2.0 ** -4 * 0.5 / 448 and d1["sa"].max() < 2.0 ** 4 * 7 / 448
