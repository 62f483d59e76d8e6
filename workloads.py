"""Seeded synthetic inputs for the fine-grained-scaled FP8 E4M3 NT GEMM.

This module is shared by the tests, the smoke check and the bench.  It draws
random fp32 data and casts it to E4M3 (or E5M2, for the dense GEMM's format
option) with per-block fp32 scales; it holds none of the GEMM's arithmetic (no
decode, no dot products, no promotion, no BF16 rounding).  The fp8 cast itself
is torch's float32 -> float8_e4m3fn / float8_e5m2 conversion (round to nearest
even); the scale arithmetic is numpy fp32 (amax / 448, or amax / 57344 for E5M2).  The oracle has its
own, independently written quantiser, and a test checks that both agree bit
for bit.

Recipe (one reading per point, all seeded, numpy PCG64 ``default_rng(seed)``):

* values: fp32 standard normal; every A 1x128 block and every B 128x128 block is
  multiplied (in fp32) by 2^u with u ~ U(-4, 4) continuous, one draw per block;
* quantisation per block: amax of |x|, scale = fp32(amax / 448) (1 if amax is 0),
  q = E4M3_RNE(clamp(fp32(x / scale), -448, 448));
* draw order: A normals (row-major, all rows incl. padding), A exponents
  (row-major [rows, Kb]); then for each group: B normals, B exponents
  ([Nb, Kb]); then masked_m (masked layout only, inclusive U{0..capacity});
* contiguous token split: expected Zipf(s) counts -- p_g ~ (g+1)^-s, floor of
  total*p_g, the remainder handed out by largest fractional part (lowest group
  first on ties) -- each segment padded up to the 128-row alignment; padding
  rows carry group index -1 and ordinary finite data;
* layouts: A [rows, K] K-major; sA fp32 [Kb, ld_sa] MN-major with ld_sa the row
  count rounded up to a multiple of 4 (padding scales 0); B [N, K] K-major;
  sB fp32 [ceil(N/128), Kb].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KBLOCK = 128
M_ALIGN = 128          # contiguous-layout segment alignment (= the kernels' M block)
E4M3_MAX = 448.0       # largest finite OCP E4M3FN value
E5M2_MAX = 57344.0     # largest finite OCP E5M2 value
FP8_MAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "dense" | "contiguous" | "masked"
    m: int = 0                     # dense rows
    n: int = 0
    k: int = 0
    groups: int = 1
    tokens: int = 0                # contiguous: valid rows before padding
    zipf_s: float = 0.0
    max_m: int = 0                 # masked capacity per group
    seed: int = 0
    extra: dict = field(default_factory=dict)


# The five workloads the library is measured on: a small all-layout sanity shape,
# a prefill-like dense shape, an under-filled small-M dense shape, a skewed
# contiguous MoE shape and a masked decode shape.
WORKLOADS = {
    "dense_m128_n128_k512": Workload("dense_m128_n128_k512", "dense", m=128, n=128, k=512),
    "dense_m4096_n7168_k7168": Workload("dense_m4096_n7168_k7168", "dense", m=4096, n=7168, k=7168),
    "dense_m256_n7168_k2048": Workload("dense_m256_n7168_k2048", "dense", m=256, n=7168, k=2048),
    "contiguous_g8_t32768_zipf1.1_n4096_k7168": Workload(
        "contiguous_g8_t32768_zipf1.1_n4096_k7168", "contiguous", n=4096, k=7168, groups=8,
        tokens=32768, zipf_s=1.1),
    "masked_g16_cap256_n4096_k7168": Workload(
        "masked_g16_cap256_n4096_k7168", "masked", n=4096, k=7168, groups=16, max_m=256),
}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def ld_sa_for(rows: int) -> int:
    return max(4, ceil_div(rows, 4) * 4)


def zipf_counts(total: int, groups: int, s: float) -> list[int]:
    """Expected Zipf(s) split of ``total`` rows over ``groups`` (largest remainder)."""
    w = [(g + 1) ** (-s) for g in range(groups)]
    z = sum(w)
    exact = [total * x / z for x in w]
    base = [math.floor(e) for e in exact]
    rest = total - sum(base)
    order = sorted(range(groups), key=lambda g: (-(exact[g] - base[g]), g))
    for g in order[:rest]:
        base[g] += 1
    return base


def padded(counts, align: int = M_ALIGN) -> list[int]:
    return [ceil_div(c, align) * align for c in counts]


def _scaled_normals(rng, rows: int, k: int, block_rows: int) -> np.ndarray:
    """fp32 N(0,1) [rows, k] with each (block_rows x 128) block times 2^U(-4,4)."""
    x = rng.standard_normal((rows, k), dtype=np.float32)
    rb, kb = ceil_div(rows, block_rows), ceil_div(k, KBLOCK)
    u = rng.uniform(-4.0, 4.0, size=(rb, kb))
    f = np.exp2(u).astype(np.float32)
    f_rows = np.repeat(f, block_rows, axis=0)[:rows]
    f_full = np.repeat(f_rows, KBLOCK, axis=1)[:, :k]
    x *= f_full
    return x


def make_fp32_operand(rows: int, k: int, block_rows: int, seed: int = 0) -> np.ndarray:
    """The recipe's fp32 values before the cast (input of the FP8 cast kernels)."""
    return _scaled_normals(np.random.default_rng(seed), rows, k, block_rows)


def _cast_fp8(y: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    dt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return t.to(dt).view(torch.uint8).numpy().copy()


def _block_scales(amax: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    amax = amax.astype(np.float32)
    s = amax / np.float32(FP8_MAX[fmt])
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quant_rows_1x128(x: np.ndarray, fmt: str = "e4m3"):
    """fp32 [rows, k] -> (FP8 bytes [rows, k], sa fp32 [Kb, ld_sa]); fmt "e4m3" or "e5m2"."""
    rows, k = x.shape
    kb = ceil_div(k, KBLOCK)
    kp = kb * KBLOCK
    xp = np.zeros((rows, kp), np.float32)
    xp[:, :k] = x
    xb = xp.reshape(rows, kb, KBLOCK)
    s = _block_scales(np.abs(xb).max(axis=2), fmt)                 # [rows, kb]
    y = np.clip(xb / s[:, :, None], -FP8_MAX[fmt], FP8_MAX[fmt]).reshape(rows, kp)[:, :k]
    q = _cast_fp8(y, fmt)
    sa = np.zeros((kb, ld_sa_for(rows)), np.float32)
    sa[:, :rows] = s.T
    return q, sa


def quant_blocks_128x128(x: np.ndarray, fmt: str = "e4m3"):
    """fp32 [n, k] -> (FP8 bytes [n, k], sb fp32 [ceil(n/128), Kb]); fmt "e4m3" or "e5m2"."""
    n, k = x.shape
    nb, kb = ceil_div(n, KBLOCK), ceil_div(k, KBLOCK)
    xp = np.zeros((nb * KBLOCK, kb * KBLOCK), np.float32)
    xp[:n, :k] = x
    xb = xp.reshape(nb, KBLOCK, kb, KBLOCK)
    s = _block_scales(np.abs(xb).max(axis=(1, 3)), fmt)             # [nb, kb]
    y = np.clip(xb / s[:, None, :, None], -FP8_MAX[fmt], FP8_MAX[fmt])
    y = y.reshape(nb * KBLOCK, kb * KBLOCK)[:n, :k]
    return _cast_fp8(y, fmt), s


def make_dense(m: int, n: int, k: int, seed: int = 0, a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> dict:
    rng = np.random.default_rng(seed)
    xa = _scaled_normals(rng, m, k, 1)
    a, sa = quant_rows_1x128(xa, a_fmt)
    del xa
    xb = _scaled_normals(rng, n, k, KBLOCK)
    b, sb = quant_blocks_128x128(xb, b_fmt)
    return {"kind": "dense", "a": a, "sa": sa, "b": b, "sb": sb, "m": m, "n": n, "k": k,
            "a_fmt": a_fmt, "b_fmt": b_fmt}


def make_contiguous(counts, n: int, k: int, seed: int = 0, align: int = M_ALIGN,
                    a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> dict:
    counts = [int(c) for c in counts]
    pads = padded(counts, align)
    m_total = sum(pads)
    m_indices = np.full(m_total, -1, np.int32)
    off = 0
    for g, (c, p) in enumerate(zip(counts, pads)):
        m_indices[off:off + c] = g
        off += p
    rng = np.random.default_rng(seed)
    xa = _scaled_normals(rng, m_total, k, 1)
    a, sa = quant_rows_1x128(xa, a_fmt)
    del xa
    G = len(counts)
    b = np.empty((G, n, k), np.uint8)
    sb = np.empty((G, ceil_div(n, KBLOCK), ceil_div(k, KBLOCK)), np.float32)
    for g in range(G):
        xb = _scaled_normals(rng, n, k, KBLOCK)
        b[g], sb[g] = quant_blocks_128x128(xb, b_fmt)
        del xb
    return {"kind": "contiguous", "a": a, "sa": sa, "b": b, "sb": sb, "m_indices": m_indices,
            "counts": counts, "m_total": m_total, "n": n, "k": k, "groups": G,
            "a_fmt": a_fmt, "b_fmt": b_fmt}


def make_masked(groups: int, max_m: int, n: int, k: int, seed: int = 0, masked_m=None,
                a_fmt: str = "e4m3", b_fmt: str = "e4m3") -> dict:
    rng = np.random.default_rng(seed)
    xa = _scaled_normals(rng, groups * max_m, k, 1)
    kb = ceil_div(k, KBLOCK)
    a = np.empty((groups, max_m, k), np.uint8)
    sa = np.zeros((groups, kb, ld_sa_for(max_m)), np.float32)
    for g in range(groups):
        q, s = quant_rows_1x128(xa[g * max_m:(g + 1) * max_m], a_fmt)
        a[g] = q
        sa[g] = s
    del xa
    b = np.empty((groups, n, k), np.uint8)
    sb = np.empty((groups, ceil_div(n, KBLOCK), kb), np.float32)
    for g in range(groups):
        xb = _scaled_normals(rng, n, k, KBLOCK)
        b[g], sb[g] = quant_blocks_128x128(xb, b_fmt)
        del xb
    mm = rng.integers(0, max_m + 1, size=groups).astype(np.int32)
    if masked_m is not None:
        mm = np.asarray(masked_m, dtype=np.int32)
    return {"kind": "masked", "a": a, "sa": sa, "b": b, "sb": sb, "masked_m": mm,
            "groups": groups, "max_m": max_m, "n": n, "k": k, "a_fmt": a_fmt, "b_fmt": b_fmt}


def make(w: Workload | str) -> dict:
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.kind == "dense":
        return make_dense(w.m, w.n, w.k, w.seed)
    if w.kind == "contiguous":
        return make_contiguous(zipf_counts(w.tokens, w.groups, w.zipf_s), w.n, w.k, w.seed)
    if w.kind == "masked":
        return make_masked(w.groups, w.max_m, w.n, w.k, w.seed)
    raise ValueError(w.kind)


# BF16 bit pattern written into masked outputs before a call: a quiet NaN with
# a payload that no fp32 -> bf16 conversion of a computed value produces.
SENTINEL_BF16 = 0x7FE5
