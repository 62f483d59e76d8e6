"""CPU oracle for the fine-grained-scaled FP8 E4M3 NT GEMM (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg are the only callers.  The HIP library never
imports, links or calls anything here, and nothing here touches a GPU.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only builds
it with gcc, loads it with ctypes and marshals numpy arrays.  What the C code
computes, and which passage of the pages each step follows, is documented at
the top of ``oracle.c``:

* ``e4m3_decode_table`` -- OCP E4M3FN value of every byte (hnwysp.cn blog
  section 4.1 fixes the +-448 range); ``e5m2_decode_table`` -- OCP E5M2, the
  other operand format the blog lists (section 2.3);
* ``e4m3_encode`` / ``bf16_encode`` -- round-to-nearest-even encoders;
* ``quantize_rows_1x128`` / ``quantize_blocks_128x128`` -- the input cast with
  per-block scales (the README's usage paragraph leaves the cast to a prior
  kernel; the granularity is the DeepSeek-V3 fine-grained scheme);
* ``gemm_fp8_nt`` / ``m_grouped_contiguous`` / ``m_grouped_masked`` -- the three
  layouts of the README ("normal", "contiguous", "masked" paragraphs); the dense
  GEMM also takes each operand's format (E4M3 or E5M2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORC_LIB: load this already-built library instead (the mutation test points the pins
# at copies of oracle.c with deliberate mistakes planted in them)
_LIB_OVERRIDE = os.environ.get("ORC_LIB")
_LIB = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
KBLOCK = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc, -O2, no fast-math,
    no FMA contraction so that every fp64 operation rounds exactly once)."""
    if _LIB_OVERRIDE:
        if force:
            raise RuntimeError("ORC_LIB is set: the oracle library is given, not built")
        return _LIB
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    compile_library(_SRC, tmp)
    os.replace(tmp, _LIB)
    return _LIB


def compile_library(src: str, out: str) -> None:
    """The one compile command of the oracle's C source (also used on planted-mistake
    copies of it by the mutation test)."""
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_OVERRIDE and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    lib.orc_e4m3_decode_table.argtypes = [P]
    lib.orc_e4m3_decode_table.restype = None
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_bf16_encode.argtypes = [ctypes.c_double]
    lib.orc_bf16_encode.restype = ctypes.c_uint16
    lib.orc_block_dot.argtypes = [P, P, I]
    lib.orc_block_dot.restype = ctypes.c_double
    lib.orc_e5m2_decode_table.argtypes = [P]
    lib.orc_e5m2_decode_table.restype = None
    lib.orc_block_dot_fmt.argtypes = [P, P, I, I, I]
    lib.orc_block_dot_fmt.restype = ctypes.c_double
    lib.orc_gemm_fp8_nt_fmt.argtypes = [P, L, P, L, P, L, P, P, L, P, I, I, I, I, I, I]
    lib.orc_gemm_fp8_nt_fmt.restype = I
    lib.orc_quantize_rows_1x128.argtypes = [P, L, I, I, P, L, P, L]
    lib.orc_quantize_rows_1x128.restype = None
    lib.orc_quantize_blocks_128x128.argtypes = [P, L, I, I, P, L, P]
    lib.orc_quantize_blocks_128x128.restype = None
    lib.orc_e5m2_encode.argtypes = [ctypes.c_double]
    lib.orc_e5m2_encode.restype = ctypes.c_uint8
    lib.orc_quantize_rows_1x128_fmt.argtypes = [P, L, I, I, P, L, P, L, I]
    lib.orc_quantize_rows_1x128_fmt.restype = None
    lib.orc_quantize_blocks_128x128_fmt.argtypes = [P, L, I, I, P, L, P, I]
    lib.orc_quantize_blocks_128x128_fmt.restype = None
    lib.orc_available_cores.argtypes = []
    lib.orc_available_cores.restype = I
    lib.orc_gemm_fp8_nt.argtypes = [P, L, P, L, P, L, P, P, L, P, I, I, I, I]
    lib.orc_gemm_fp8_nt.restype = I
    lib.orc_m_grouped_contiguous.argtypes = [P, P, L, P, P, P, P, P, I, I, I, I, I]
    lib.orc_m_grouped_contiguous.restype = I
    lib.orc_m_grouped_masked.argtypes = [P, P, L, P, P, P, P, P, I, I, I, I, I]
    lib.orc_m_grouped_masked.restype = I
    lib.orc_m_grouped_contiguous_fmt.argtypes = [P, P, L, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.orc_m_grouped_contiguous_fmt.restype = I
    lib.orc_m_grouped_masked_fmt.argtypes = [P, P, L, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.orc_m_grouped_masked_fmt.restype = I
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint8:
        a = a.view(np.uint8)
    return np.ascontiguousarray(a)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def available_cores() -> int:
    """Cores this process may run on (sched_getaffinity)."""
    return int(_load().orc_available_cores())


def e4m3_decode_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    _load().orc_e4m3_decode_table(_ptr(out))
    return out


def e5m2_decode_table() -> np.ndarray:
    out = np.empty(256, dtype=np.float64)
    _load().orc_e5m2_decode_table(_ptr(out))
    return out


FORMATS = {"e4m3": 0, "e5m2": 1}


def e4m3_encode(x: float) -> int:
    return int(_load().orc_e4m3_encode(float(x)))


def e5m2_encode(x: float) -> int:
    return int(_load().orc_e5m2_encode(float(x)))


def bf16_encode(x: float) -> int:
    return int(_load().orc_bf16_encode(float(x)))


def block_dot(a, b) -> float:
    a, b = _u8(a), _u8(b)
    assert a.shape == b.shape and a.ndim == 1
    return float(_load().orc_block_dot(_ptr(a), _ptr(b), int(a.size)))


def block_dot_fmt(a, b, a_fmt="e4m3", b_fmt="e4m3") -> float:
    """Block dot product with each operand in its own format, summed exactly."""
    a, b = _u8(a), _u8(b)
    assert a.shape == b.shape and a.ndim == 1
    return float(_load().orc_block_dot_fmt(_ptr(a), _ptr(b), int(a.size), FORMATS[a_fmt], FORMATS[b_fmt]))


def quantize_rows_1x128(x, fmt="e4m3"):
    """fp32 [m, k] -> (FP8 bytes [m, k], sa fp32 [ceil(k/128), m]) (MN-major scales);
    fmt "e4m3" (scale amax/448) or "e5m2" (scale amax/57344)."""
    x = _f32(x)
    m, k = x.shape
    kb = -(-k // KBLOCK)
    q = np.empty((m, k), dtype=np.uint8)
    sa = np.empty((kb, m), dtype=np.float32)
    if fmt == "e4m3":
        _load().orc_quantize_rows_1x128(_ptr(x), k, m, k, _ptr(q), k, _ptr(sa), m)
    else:
        _load().orc_quantize_rows_1x128_fmt(_ptr(x), k, m, k, _ptr(q), k, _ptr(sa), m, FORMATS[fmt])
    return q, sa


def quantize_blocks_128x128(x, fmt="e4m3"):
    """fp32 [n, k] -> (FP8 bytes [n, k], sb fp32 [ceil(n/128), ceil(k/128)]); fmt as
    in quantize_rows_1x128."""
    x = _f32(x)
    n, k = x.shape
    q = np.empty((n, k), dtype=np.uint8)
    sb = np.empty((-(-n // KBLOCK), -(-k // KBLOCK)), dtype=np.float32)
    if fmt == "e4m3":
        _load().orc_quantize_blocks_128x128(_ptr(x), k, n, k, _ptr(q), k, _ptr(sb))
    else:
        _load().orc_quantize_blocks_128x128_fmt(_ptr(x), k, n, k, _ptr(q), k, _ptr(sb), FORMATS[fmt])
    return q, sb


def gemm_fp8_nt(a, sa, b, sb, *, d_init=None, want_acc=False, nthreads=0, a_fmt="e4m3", b_fmt="e4m3"):
    """Dense NT GEMM.  a: FP8 [m, k]; sa: fp32 [Kb, ld_sa>=m] (MN-major);
    b: FP8 [n, k]; sb: fp32 [ceil(n/128), Kb]; each operand E4M3 or E5M2.  Returns
    BF16 bits uint16 [m, n] (and the fp64 accumulator when ``want_acc``)."""
    a, b, sa, sb = _u8(a), _u8(b), _f32(sa), _f32(sb)
    m, k = a.shape
    n = b.shape[0]
    assert b.shape[1] == k and sa.shape[0] == -(-k // KBLOCK) and sa.shape[1] >= m
    assert sb.shape == (-(-n // KBLOCK), -(-k // KBLOCK))
    d = np.zeros((m, n), np.uint16) if d_init is None else np.array(d_init, np.uint16, copy=True)
    acc = np.full((m, n), np.nan) if want_acc else None
    if a_fmt == "e4m3" and b_fmt == "e4m3":
        _load().orc_gemm_fp8_nt(_ptr(a), k, _ptr(sa), sa.shape[1], _ptr(b), k, _ptr(sb),
                                _ptr(d), n, _ptr(acc), m, n, k, int(nthreads))
    else:
        _load().orc_gemm_fp8_nt_fmt(_ptr(a), k, _ptr(sa), sa.shape[1], _ptr(b), k, _ptr(sb),
                                    _ptr(d), n, _ptr(acc), m, n, k, FORMATS[a_fmt], FORMATS[b_fmt],
                                    int(nthreads))
    return (d, acc) if want_acc else d


def m_grouped_contiguous(a, sa, b, sb, m_indices, *, d_init=None, want_acc=False, nthreads=0,
                         a_fmt="e4m3", b_fmt="e4m3"):
    """a: FP8 [m_total, k]; sa: fp32 [Kb, ld_sa>=m_total]; b: FP8 [G, n, k];
    sb: fp32 [G, ceil(n/128), Kb]; m_indices: int32 [m_total] (group or -1); each
    operand E4M3 or E5M2.  Rows with -1 keep ``d_init`` (zeros by default)."""
    a, b, sa, sb = _u8(a), _u8(b), _f32(sa), _f32(sb)
    mi = np.ascontiguousarray(np.asarray(m_indices, dtype=np.int32))
    m_total, k = a.shape
    g, n, _ = b.shape
    assert mi.shape == (m_total,) and sb.shape == (g, -(-n // KBLOCK), -(-k // KBLOCK))
    assert mi.max(initial=-1) < g
    d = np.zeros((m_total, n), np.uint16) if d_init is None else np.array(d_init, np.uint16, copy=True)
    acc = np.full((m_total, n), np.nan) if want_acc else None
    if a_fmt == "e4m3" and b_fmt == "e4m3":
        _load().orc_m_grouped_contiguous(_ptr(a), _ptr(sa), sa.shape[1], _ptr(b), _ptr(sb),
                                         _ptr(d), _ptr(acc), _ptr(mi), m_total, n, k, g, int(nthreads))
    else:
        _load().orc_m_grouped_contiguous_fmt(_ptr(a), _ptr(sa), sa.shape[1], _ptr(b), _ptr(sb),
                                             _ptr(d), _ptr(acc), _ptr(mi), m_total, n, k, g,
                                             FORMATS[a_fmt], FORMATS[b_fmt], int(nthreads))
    return (d, acc) if want_acc else d


def m_grouped_masked(a, sa, b, sb, masked_m, *, d_init=None, want_acc=False, nthreads=0,
                     a_fmt="e4m3", b_fmt="e4m3"):
    """a: FP8 [G, max_m, k]; sa: fp32 [G, Kb, ld_sa>=max_m]; b: FP8 [G, n, k];
    sb: fp32 [G, ceil(n/128), Kb]; masked_m: int32 [G]; each operand E4M3 or
    E5M2.  Rows >= masked_m[g] keep ``d_init`` (zeros by default)."""
    a, b, sa, sb = _u8(a), _u8(b), _f32(sa), _f32(sb)
    mm = np.ascontiguousarray(np.asarray(masked_m, dtype=np.int32))
    g, max_m, k = a.shape
    n = b.shape[1]
    assert b.shape == (g, n, k) and mm.shape == (g,)
    assert sa.shape[:2] == (g, -(-k // KBLOCK)) and sa.shape[2] >= max_m
    d = np.zeros((g, max_m, n), np.uint16) if d_init is None else np.array(d_init, np.uint16, copy=True)
    acc = np.full((g, max_m, n), np.nan) if want_acc else None
    if a_fmt == "e4m3" and b_fmt == "e4m3":
        _load().orc_m_grouped_masked(_ptr(a), _ptr(sa), sa.shape[2], _ptr(b), _ptr(sb),
                                     _ptr(d), _ptr(acc), _ptr(mm), g, max_m, n, k, int(nthreads))
    else:
        _load().orc_m_grouped_masked_fmt(_ptr(a), _ptr(sa), sa.shape[2], _ptr(b), _ptr(sb),
                                         _ptr(d), _ptr(acc), _ptr(mm), g, max_m, n, k,
                                         FORMATS[a_fmt], FORMATS[b_fmt], int(nthreads))
    return (d, acc) if want_acc else d
