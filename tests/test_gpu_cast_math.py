"""GPU evidence for the FP8 casts' fast quotient: the casts' own device functions
(dg_cast_math.h, run through the test probe tests/hip_probe/libcastprobe.so) against
the IEEE single-precision division, bit for bit.

* rcp_exact(s) equals 1/s for EVERY fp32 scale the fast path admits (2^-64 <= s <
  2^125); the hardware reciprocal estimate alone does not, so the comparison can fail.
* div_fast(x, s, rcp_exact(s)) equals x/s for ~4300 scales spread over every binade the
  casts can produce, each with x at every value and rounding tie of the FP8 formats
  times s and the fp32 neighbours of those products, plus 4096 pseudo-random x in
  [-FMAX*s, FMAX*s].
"""
import ctypes
import os

import numpy as np
import pytest

from tests.gpu_support import require_gpu, say

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "hip_probe", "libcastprobe.so")


@pytest.fixture(scope="module")
def probe():
    require_gpu()
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: build it with tests/hip_probe/build.py (build() does)")
    lib = ctypes.CDLL(PROBE)
    lib.probe_rcp_exact.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32)]
    lib.probe_rcp_exact.restype = ctypes.c_int
    lib.probe_div_fast.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_float, ctypes.POINTER(ctypes.c_ulonglong),
                                   ctypes.POINTER(ctypes.c_uint32)]
    lib.probe_div_fast.restype = ctypes.c_int
    return lib


def f32_bits(x: float) -> int:
    return int(np.array([x], np.float32).view(np.uint32)[0])


def rcp(lib, lo, hi, raw=0):
    bad, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
    rc = lib.probe_rcp_exact(lo, hi, raw, ctypes.byref(bad), ctypes.byref(first))
    assert rc == 0, f"probe failed with HIP error {rc}"
    return bad.value, first.value


def test_rcp_exact_for_every_fast_path_scale(probe):
    lo, hi = f32_bits(2.0 ** -64), f32_bits(2.0 ** 125) - 1
    say(f"rcp_exact over fp32 bit patterns 0x{lo:08x}..0x{hi:08x} ({hi - lo + 1} values)")
    bad, first = rcp(probe, lo, hi)
    assert bad == 0, f"{bad} scales differ from the IEEE reciprocal, first 0x{first:08x}"


def test_rcp_probe_notices_the_raw_estimate(probe):
    lo = f32_bits(1.0)
    bad, _ = rcp(probe, lo, lo + (1 << 23) - 1, raw=1)
    assert bad > 0


def _multipliers(fmt):
    """Every value and rounding tie of the format in [-FMAX, FMAX] (normal and
    subnormal), quotients below 2^-20 left out: those are far under half the smallest
    FP8 subnormal, so any quotient there encodes as a zero of the right sign."""
    vals = [0.0]
    if fmt == "e4m3":
        for e in range(-9, 9):
            for m in range(16):
                for frac in (0.0, 0.5):
                    vals.append(2.0 ** e * (1 + (m + frac) / 8) if e >= -6 else (m + frac) * 2.0 ** -9)
        fmax = 448.0
    else:
        for e in range(-17, 16):
            for m in range(8):
                for frac in (0.0, 0.5):
                    vals.append(2.0 ** e * (1 + (m + frac) / 4) if e >= -14 else (m + frac) * 2.0 ** -16)
        fmax = 57344.0
    v = np.array(sorted(set(vals)), np.float64)
    v = v[(v == 0) | ((v >= 2.0 ** -20) & (v <= fmax))]
    return np.concatenate([v, -v[v > 0]]).astype(np.float32), fmax


def _scales(fmax, seed):
    """24 significands (1, the largest, 22 random) at every binade from 2^-64 up to
    nearly the largest scale a finite amax gives (FLT_MAX / FMAX; kept 2^-20 below it so
    that FMAX * s and its fp32 neighbours stay finite)."""
    rng = np.random.default_rng(seed)
    top = float(np.finfo(np.float32).max) / fmax * (1 - 2.0 ** -20)
    out = []
    for e in range(-64, 128):
        sig = np.concatenate([[1.0, 2.0 - 2.0 ** -23], 1.0 + rng.integers(0, 1 << 23, 22) / 2.0 ** 23])
        s = (sig * 2.0 ** e).astype(np.float32)
        out.append(s[(s >= 2.0 ** -64) & (s <= top)])
    return np.concatenate(out).astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_div_fast_is_the_ieee_quotient(probe, fmt):
    mult, fmax = _multipliers(fmt)
    scales = _scales(fmax, seed=11 if fmt == "e4m3" else 12)
    say(f"div_fast {fmt}: {scales.size} scales x ({3 * mult.size} tie-grid + 4096 random) values")
    bad, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
    rc = probe.probe_div_fast(scales.ctypes.data, scales.size, mult.ctypes.data, mult.size, 4096, fmax,
                              ctypes.byref(bad), ctypes.byref(first))
    assert rc == 0, f"probe failed with HIP error {rc}"
    assert bad.value == 0, f"{bad.value} quotients differ; first at scale {scales[first.value]!r}"
