"""Helpers shared by the GPU parity tests, the smoke check and the bench: device
upload of the seeded workloads, the acceptance check against the oracle's BF16
output, and row sampling for full-size shapes."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W

# Acceptance bar for floating-point parity (per element and whole output).  The
# oracle's result is exact up to one fp64 rounding per K block; the kernels add
# fp32 promotion and the MFMA's own summation, so a small relative error plus a
# floor tied to the output's scale is allowed, and the output as a whole must
# match to 1e-3 in normalised Frobenius norm (BF16 rounding alone of an exact
# result against its BF16 image is already ~2^-9 per element).
REL_TOL = 2.0 ** -7
ABS_TOL_FRAC = 2.0 ** -10
FRO_TOL = 1e-3


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible gfx950 device")
    return torch.device("cuda:0")


def to_dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def sentinel_like(shape):
    import torch
    return torch.full(shape, W.SENTINEL_BF16, dtype=torch.int16, device="cuda:0")


def bits(t) -> np.ndarray:
    """BF16 output (as bfloat16 or its int16 bit pattern) -> uint16 bits on the host."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def check_values(gpu_bits: np.ndarray, ref_bits: np.ndarray, where: str = "") -> float:
    """Per element |g - r| <= 2^-7 |r| + 2^-10 max|r|, no NaN/Inf, and normalised
    Frobenius error <= 1e-3.  Returns the Frobenius error."""
    assert gpu_bits.shape == ref_bits.shape, (gpu_bits.shape, ref_bits.shape)
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    assert np.isfinite(r).all(), f"{where}: oracle produced non-finite values"
    nonfinite = ~np.isfinite(g)
    assert not nonfinite.any(), f"{where}: {nonfinite.sum()} non-finite outputs, first at {np.argwhere(nonfinite)[0]}"
    mx = float(np.abs(r).max()) if r.size else 0.0
    err = np.abs(g - r)
    bad = err > REL_TOL * np.abs(r) + ABS_TOL_FRAC * mx
    assert not bad.any(), (f"{where}: {bad.sum()} of {bad.size} elements out of tolerance; first at "
                           f"{np.argwhere(bad)[0]}: gpu {g[tuple(np.argwhere(bad)[0])]} ref {r[tuple(np.argwhere(bad)[0])]}")
    den = float(np.linalg.norm(r))
    fro = float(np.linalg.norm(g - r)) / den if den > 0 else float(np.linalg.norm(g))
    assert fro <= FRO_TOL, f"{where}: normalised Frobenius error {fro:.3e} > {FRO_TOL}"
    return fro


def sample_rows(rows: int, block: int, count: int, seed: int = 123) -> np.ndarray:
    """First and last row of several row blocks plus random rows, sorted, unique."""
    rng = np.random.default_rng(seed)
    picks = {0, rows - 1}
    nblk = -(-rows // block)
    for b in rng.choice(nblk, size=min(nblk, max(1, count // 4)), replace=False):
        picks.add(int(b) * block)
        picks.add(min(rows - 1, int(b) * block + block - 1))
    while len(picks) < min(count, rows):
        picks.add(int(rng.integers(rows)))
    return np.array(sorted(picks), dtype=np.int64)


def upload(data: dict) -> dict:
    out = {}
    for key in ("a", "sa", "b", "sb", "m_indices", "masked_m"):
        if key in data:
            out[key] = to_dev(data[key])
    return out
