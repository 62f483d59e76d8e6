"""Python binding of libdg.so: fine-grained-scaled FP8 E4M3 NT GEMM for MI355X.

Argument marshalling only.  Each function has the name of the C entry point it
calls (see ``include/dg.h`` for the operation, layouts and error behaviour),
takes torch tensors that already live on the GPU, passes their device pointers
and torch's current HIP stream, and raises :class:`DGError` on a non-zero
status.  All arithmetic runs in the library's gfx950 kernels; there is no other
implementation here and no fallback: if ``libdg.so`` is missing the import of
the library fails with an error.

Tensor conventions (the README's NT format and layouts):
  A  ``torch.float8_e4m3fn`` (or uint8 holding E4M3 bytes), [M, K] contiguous rows
  sA ``torch.float32`` [K/128, ld_sa] (MN-major: one row per K block)
  B  E4M3 [N, K]; grouped [G, N, K]
  sB ``torch.float32`` [ceil(N/128), K/128]; grouped [G, ceil(N/128), K/128]
  D  ``torch.bfloat16`` (or int16/uint16 bits) [M, N]
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK = 0
DG_ERR_INVALID_ARG = -1
DG_ERR_UNSUPPORTED = -2
DG_ERR_MISALIGNED = -3
DG_ERR_HIP = -4

_lib = None


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdg.so (built by ``fp8_block_scaled_e4m3_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libdg.so not found at {path}; run `python -m fp8_block_scaled_e4m3_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P, L, I = ctypes.c_void_p, ctypes.c_long, ctypes.c_int
    lib.dg_status_string.argtypes = [I]
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_get_m_alignment.argtypes = []
    lib.dg_get_m_alignment.restype = I
    lib.dg_set_num_cus.argtypes = [I]
    lib.dg_set_num_cus.restype = I
    lib.dg_get_num_cus.argtypes = []
    lib.dg_get_num_cus.restype = I
    lib.dg_gemm_fp8_nt.argtypes = [P, L, P, L, P, L, P, P, L, I, I, I, P]
    lib.dg_gemm_fp8_nt.restype = I
    lib.dg_gemm_fp8_nt_fmt.argtypes = [P, L, P, L, P, L, P, P, L, I, I, I, I, I, P]
    lib.dg_gemm_fp8_nt_fmt.restype = I
    lib.dg_m_grouped_gemm_fp8_contiguous.argtypes = [P, P, L, P, P, P, P, I, I, I, I, P]
    lib.dg_m_grouped_gemm_fp8_contiguous.restype = I
    lib.dg_m_grouped_gemm_fp8_masked.argtypes = [P, P, L, P, P, P, P, I, I, I, I, P]
    lib.dg_m_grouped_gemm_fp8_masked.restype = I
    lib.dg_m_grouped_gemm_fp8_contiguous_fmt.argtypes = [P, P, L, P, P, P, P, I, I, I, I, I, I, P]
    lib.dg_m_grouped_gemm_fp8_contiguous_fmt.restype = I
    lib.dg_m_grouped_gemm_fp8_masked_fmt.argtypes = [P, P, L, P, P, P, P, I, I, I, I, I, I, P]
    lib.dg_m_grouped_gemm_fp8_masked_fmt.restype = I
    lib.dg_quantize_fp8_1x128.argtypes = [P, I, L, I, I, P, L, P, L, P]
    lib.dg_quantize_fp8_1x128.restype = I
    lib.dg_quantize_fp8_128x128.argtypes = [P, I, L, I, I, P, L, P, P]
    lib.dg_quantize_fp8_1x128_fmt.argtypes = [P, I, L, I, I, P, L, P, L, I, P]
    lib.dg_quantize_fp8_1x128_fmt.restype = I
    lib.dg_quantize_fp8_128x128_fmt.argtypes = [P, I, L, I, I, P, L, P, I, P]
    lib.dg_quantize_fp8_128x128_fmt.restype = I
    lib.dg_quantize_fp8_128x128.restype = I
    lib.dg_set_kernel_config.argtypes = [I]
    lib.dg_set_kernel_config.restype = I
    lib.dg_kernel_config_info.argtypes = [I, P]
    lib.dg_kernel_config_info.restype = I
    lib.dg_plan_tiles.argtypes = [I, I, I, I, P, I, P, I, P, P]
    lib.dg_plan_tiles.restype = I
    lib.dg_describe_launch.argtypes = [I, I, I, I, I, I, P]
    lib.dg_describe_launch.restype = I
    lib.dg_get_aligned_ld_sa.argtypes = [L]
    lib.dg_get_aligned_ld_sa.restype = L
    lib.dg_transform_sa_mn_major.argtypes = [P, L, P, L, I, I, I, P]
    lib.dg_transform_sa_mn_major.restype = I
    lib.dg_check_contiguous_layout.argtypes = [P, I, I, P]
    lib.dg_check_contiguous_layout.restype = I
    _lib = lib
    return lib


def dg_status_string(status: int) -> str:
    return load_library().dg_status_string(int(status)).decode()


status_string = dg_status_string


def _check(status: int, where: str) -> None:
    if status != DG_OK:
        raise DGError(status, where)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, name: str, dtypes, ndim: int):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dimension")
    return ctypes.c_void_p(t.data_ptr())


def _fp8_types():
    import torch
    return (torch.float8_e4m3fn, torch.uint8)


def _fp8_any_types():
    import torch
    return (torch.float8_e4m3fn, torch.float8_e5m2, torch.uint8)


DG_FMT_E4M3, DG_FMT_E5M2 = 0, 1
_FMT_NAMES = {"e4m3": DG_FMT_E4M3, "e5m2": DG_FMT_E5M2}


def _fmt_of(t, given):
    """Operand format: a float8 dtype carries it (float8_e5m2 -> E5M2, float8_e4m3fn ->
    E4M3); for uint8 bytes ``given`` ("e4m3" / "e5m2") decides, E4M3 when None."""
    import torch
    from_dtype = {torch.float8_e5m2: DG_FMT_E5M2, torch.float8_e4m3fn: DG_FMT_E4M3}.get(t.dtype)
    if given is None:
        return DG_FMT_E4M3 if from_dtype is None else from_dtype
    if given not in _FMT_NAMES:
        raise ValueError(f"unknown FP8 format {given!r}")
    if from_dtype is not None and from_dtype != _FMT_NAMES[given]:
        raise ValueError(f"format {given!r} does not match dtype {t.dtype}")
    return _FMT_NAMES[given]


def _f32():
    import torch
    return (torch.float32,)


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def dg_get_m_alignment() -> int:
    return int(load_library().dg_get_m_alignment())


def dg_set_num_cus(n: int) -> None:
    _check(load_library().dg_set_num_cus(int(n)), "dg_set_num_cus")


def dg_get_num_cus() -> int:
    v = int(load_library().dg_get_num_cus())
    if v < 0:
        raise DGError(v, "dg_get_num_cus")
    return v


def dg_gemm_fp8_nt(a, sa, b, sb, d, stream=None) -> None:
    """D[m, n] = bf16(sum_kb sA[kb, m] * sB[n // 128, kb] * A[m, kb-block] . B[n, kb-block]).
    E4M3 operands; a tensor of dtype float8_e5m2 is taken as E5M2 (see dg_gemm_fp8_nt_fmt)."""
    dg_gemm_fp8_nt_fmt(a, sa, b, sb, d, None, None, stream)


def dg_gemm_fp8_nt_fmt(a, sa, b, sb, d, a_fmt=None, b_fmt=None, stream=None) -> None:
    """The dense GEMM with each operand E4M3 or E5M2 ("e4m3" / "e5m2"; float8 tensors
    carry their format in the dtype, uint8 bytes default to E4M3)."""
    m, k = a.shape
    n = b.shape[0]
    pa = _dev(a, "a", _fp8_any_types(), 2)
    psa = _dev(sa, "sa", _f32(), 2)
    pb = _dev(b, "b", _fp8_any_types(), 2)
    psb = _dev(sb, "sb", _f32(), 2)
    pd = _dev(d, "d", _bf16_types(), 2)
    fa, fb = _fmt_of(a, a_fmt), _fmt_of(b, b_fmt)
    if b.shape[1] != k or tuple(d.shape) != (m, n):
        raise ValueError(f"shape mismatch: a {tuple(a.shape)}, b {tuple(b.shape)}, d {tuple(d.shape)}")
    if sa.shape[0] != -(-k // 128) or sa.shape[1] < m or sb.shape[1] != -(-k // 128) or sb.shape[0] != -(-n // 128):
        raise ValueError(f"scale shape mismatch: sa {tuple(sa.shape)}, sb {tuple(sb.shape)}")
    if not sb.is_contiguous():
        raise ValueError("sb must be contiguous")
    _check(load_library().dg_gemm_fp8_nt_fmt(pa, a.stride(0), psa, sa.stride(0), pb, b.stride(0), psb,
                                             pd, d.stride(0), m, n, k, fa, fb, _stream(stream)),
           "dg_gemm_fp8_nt_fmt")


def dg_m_grouped_gemm_fp8_contiguous(a, sa, b, sb, d, m_indices, stream=None) -> None:
    """Contiguous M-grouped GEMM; rows with m_indices == -1 are not written.  E4M3
    operands; float8_e5m2 tensors are taken as E5M2 (see the _fmt call)."""
    dg_m_grouped_gemm_fp8_contiguous_fmt(a, sa, b, sb, d, m_indices, None, None, stream)


def dg_m_grouped_gemm_fp8_contiguous_fmt(a, sa, b, sb, d, m_indices, a_fmt=None, b_fmt=None, stream=None) -> None:
    """The contiguous M-grouped GEMM with each operand E4M3 or E5M2 (as dg_gemm_fp8_nt_fmt)."""
    import torch
    m_total, k = a.shape
    g, n, _ = b.shape
    pa = _dev(a, "a", _fp8_any_types(), 2)
    psa = _dev(sa, "sa", _f32(), 2)
    pb = _dev(b, "b", _fp8_any_types(), 3)
    psb = _dev(sb, "sb", _f32(), 3)
    pd = _dev(d, "d", _bf16_types(), 2)
    pmi = _dev(m_indices, "m_indices", (torch.int32,), 1)
    fa, fb = _fmt_of(a, a_fmt), _fmt_of(b, b_fmt)
    for t, nm in ((a, "a"), (b, "b"), (sb, "sb"), (d, "d"), (m_indices, "m_indices")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if tuple(d.shape) != (m_total, n) or b.shape[2] != k or m_indices.shape[0] != m_total:
        raise ValueError("shape mismatch")
    if tuple(sb.shape) != (g, -(-n // 128), -(-k // 128)) or sa.shape[0] != -(-k // 128) or sa.shape[1] < m_total:
        raise ValueError("scale shape mismatch")
    _check(load_library().dg_m_grouped_gemm_fp8_contiguous_fmt(pa, psa, sa.stride(0), pb, psb, pd, pmi,
                                                               m_total, n, k, g, fa, fb, _stream(stream)),
           "dg_m_grouped_gemm_fp8_contiguous_fmt")


def dg_m_grouped_gemm_fp8_masked(a, sa, b, sb, d, masked_m, stream=None) -> None:
    """Masked M-grouped GEMM; rows >= masked_m[g] of d are never written.  E4M3
    operands; float8_e5m2 tensors are taken as E5M2 (see the _fmt call)."""
    dg_m_grouped_gemm_fp8_masked_fmt(a, sa, b, sb, d, masked_m, None, None, stream)


def dg_m_grouped_gemm_fp8_masked_fmt(a, sa, b, sb, d, masked_m, a_fmt=None, b_fmt=None, stream=None) -> None:
    """The masked M-grouped GEMM with each operand E4M3 or E5M2 (as dg_gemm_fp8_nt_fmt)."""
    import torch
    g, max_m, k = a.shape
    n = b.shape[1]
    pa = _dev(a, "a", _fp8_any_types(), 3)
    psa = _dev(sa, "sa", _f32(), 3)
    pb = _dev(b, "b", _fp8_any_types(), 3)
    psb = _dev(sb, "sb", _f32(), 3)
    pd = _dev(d, "d", _bf16_types(), 3)
    pmm = _dev(masked_m, "masked_m", (torch.int32,), 1)
    fa, fb = _fmt_of(a, a_fmt), _fmt_of(b, b_fmt)
    for t, nm in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb"), (d, "d"), (masked_m, "masked_m")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if tuple(b.shape) != (g, n, k) or tuple(d.shape) != (g, max_m, n) or masked_m.shape[0] != g:
        raise ValueError("shape mismatch")
    if tuple(sb.shape) != (g, -(-n // 128), -(-k // 128)) or sa.shape[:2] != (g, -(-k // 128)):
        raise ValueError("scale shape mismatch")
    _check(load_library().dg_m_grouped_gemm_fp8_masked_fmt(pa, psa, sa.shape[2], pb, psb, pd, pmm,
                                                           g, max_m, n, k, fa, fb, _stream(stream)),
           "dg_m_grouped_gemm_fp8_masked_fmt")


def _quant_args(x, q, name):
    import torch
    if x.dtype == torch.float32:
        dt = 0
    elif x.dtype in (torch.bfloat16,):
        dt = 1
    else:
        raise TypeError(f"{name}: x must be float32 or bfloat16, got {x.dtype}")
    px = _dev(x, "x", (torch.float32, torch.bfloat16), 2)
    pq = _dev(q, "q", _fp8_any_types(), 2)
    if tuple(q.shape) != tuple(x.shape):
        raise ValueError(f"{name}: q shape {tuple(q.shape)} != x shape {tuple(x.shape)}")
    return dt, px, pq


def dg_quantize_fp8_1x128(x, q, sa, stream=None) -> None:
    """Cast x [rows, k] (fp32/bf16) to E4M3 q with per-1x128 scales sa [k/128, ld_sa]
    (MN-major); a float8_e5m2 q receives E5M2 codes (see the _fmt call)."""
    dg_quantize_fp8_1x128_fmt(x, q, sa, None, stream)


def dg_quantize_fp8_1x128_fmt(x, q, sa, q_fmt=None, stream=None) -> None:
    """The 1x128 cast with the output format "e4m3" or "e5m2" (scale amax/448 or amax/57344)."""
    rows, k = x.shape
    dt, px, pq = _quant_args(x, q, "dg_quantize_fp8_1x128_fmt")
    fq = _fmt_of(q, q_fmt)
    psa = _dev(sa, "sa", _f32(), 2)
    if sa.shape[0] != -(-k // 128) or sa.shape[1] < rows:
        raise ValueError(f"sa shape {tuple(sa.shape)} does not fit rows={rows}, k={k}")
    _check(load_library().dg_quantize_fp8_1x128_fmt(px, dt, x.stride(0), rows, k, pq, q.stride(0), psa,
                                                    sa.stride(0), fq, _stream(stream)), "dg_quantize_fp8_1x128_fmt")


def dg_quantize_fp8_128x128(x, q, sb, stream=None) -> None:
    """Cast x [rows, k] (fp32/bf16) to E4M3 q with per-128x128 scales sb [ceil(rows/128), k/128];
    a float8_e5m2 q receives E5M2 codes (see the _fmt call)."""
    dg_quantize_fp8_128x128_fmt(x, q, sb, None, stream)


def dg_quantize_fp8_128x128_fmt(x, q, sb, q_fmt=None, stream=None) -> None:
    """The 128x128 cast with the output format "e4m3" or "e5m2"."""
    rows, k = x.shape
    dt, px, pq = _quant_args(x, q, "dg_quantize_fp8_128x128_fmt")
    fq = _fmt_of(q, q_fmt)
    psb = _dev(sb, "sb", _f32(), 2)
    if tuple(sb.shape) != (-(-rows // 128), -(-k // 128)) or not sb.is_contiguous():
        raise ValueError(f"sb must be contiguous [{-(-rows // 128)}, {-(-k // 128)}], got {tuple(sb.shape)}")
    _check(load_library().dg_quantize_fp8_128x128_fmt(px, dt, x.stride(0), rows, k, pq, q.stride(0), psb, fq,
                                                      _stream(stream)), "dg_quantize_fp8_128x128_fmt")


def dg_get_aligned_ld_sa(rows: int) -> int:
    """Smallest leading dimension of an MN-major sA for ``rows`` rows that the GEMMs and
    the 1x128 cast accept (rows rounded up to a multiple of 4)."""
    v = int(load_library().dg_get_aligned_ld_sa(int(rows)))
    if v < 0:
        raise DGError(v, "dg_get_aligned_ld_sa")
    return v


def dg_transform_sa_mn_major(sa_in, sa_out=None, stream=None):
    """Per-row scales stored row-major, ``sa_in`` [rows, K/128] (or [G, rows, K/128]),
    to the MN-major layout the GEMMs read, [K/128, ld_sa] (or [G, K/128, ld_sa]) with
    ld_sa = dg_get_aligned_ld_sa(rows).  Returns ``sa_out`` (allocated by torch when
    not given; its padding columns are then zero)."""
    import torch
    squeeze = sa_in.dim() == 2
    x = sa_in.unsqueeze(0) if squeeze else sa_in
    _dev(x, "sa_in", _f32(), 3)
    g, rows, kb = x.shape
    if g > 1 and x.stride(0) != rows * x.stride(1):
        raise ValueError("sa_in groups must be stacked contiguously ([G, rows, ld_in] with stride rows*ld_in)")
    ld = dg_get_aligned_ld_sa(rows)
    if sa_out is None:
        sa_out = torch.zeros((g, kb, ld) if not squeeze else (kb, ld), dtype=torch.float32, device=x.device)
    y = sa_out.unsqueeze(0) if squeeze else sa_out
    _dev(y, "sa_out", _f32(), 3)
    if tuple(y.shape[:2]) != (g, kb) or y.shape[2] < rows or not y.is_contiguous():
        raise ValueError(f"sa_out must be contiguous [{g}, {kb}, >= {rows}], got {tuple(y.shape)}")
    _check(load_library().dg_transform_sa_mn_major(ctypes.c_void_p(x.data_ptr()), x.stride(1),
                                                   ctypes.c_void_p(y.data_ptr()), y.shape[2], rows, kb, g,
                                                   _stream(stream)), "dg_transform_sa_mn_major")
    return sa_out


def dg_check_contiguous_layout(m_indices, num_groups: int):
    """Check the contiguous layout's precondition on a host copy of m_indices (numpy or
    CPU tensor).  Returns None when it holds, else the first offending row."""
    import numpy as np
    mi = np.ascontiguousarray(np.asarray(m_indices, dtype=np.int32))
    bad = ctypes.c_int(-1)
    r = load_library().dg_check_contiguous_layout(mi.ctypes.data_as(ctypes.c_void_p), int(mi.size),
                                                  int(num_groups), ctypes.byref(bad))
    if r == DG_OK:
        return None
    if bad.value < 0:
        raise DGError(r, "dg_check_contiguous_layout")
    return int(bad.value)


# ---- the README's Python names ("deepseek-ai/deepgemm: clean and efficient FP8 GEMM
# kernels", usage and utility paragraphs): the same calls, with operands passed as
# (data, scale) pairs and the LHS scales as the README lays them out -- a [M, K/128]
# tensor stored column-major (MN-major) with a 16-byte-aligned leading dimension, as
# get_col_major_tma_aligned_tensor returns it.  Argument marshalling only.
def _lhs_scales_mn_major(s, name):
    """[.., M, K/128] column-major LHS scales -> the [.., K/128, ld] MN-major view the
    dg_ calls take (no copy)."""
    if s.stride(-2) != 1:
        raise ValueError(f"{name}: the LHS scales must be column-major (MN-major): "
                         "make them with get_col_major_tma_aligned_tensor")
    return s.transpose(-1, -2)


def set_num_sms(n: int) -> None:
    """Cap the compute units the GEMMs may occupy (0: all)."""
    dg_set_num_cus(n)


def get_num_sms() -> int:
    return dg_get_num_cus()


def get_m_alignment_for_contiguous_layout() -> int:
    return dg_get_m_alignment()


def get_tma_aligned_size(x: int, element_size: int) -> int:
    """``x`` elements of ``element_size`` bytes rounded up to a whole number of 16-byte
    units (the leading dimension an MN-major scale tensor needs)."""
    if element_size <= 0 or 16 % element_size:
        raise ValueError("element_size must divide 16")
    per = 16 // element_size
    return -(-int(x) // per) * per


def get_col_major_tma_aligned_tensor(x):
    """fp32 scales ``x`` [M, K/128] (or [G, M, K/128]) -> the same values in a new tensor
    of the same shape stored column-major with a 16-byte-aligned leading dimension (the
    GPU transform kernel writes it)."""
    squeeze = x.dim() == 2
    xs = x.unsqueeze(0) if squeeze else x
    if not xs.is_contiguous():
        xs = xs.contiguous()
    store = dg_transform_sa_mn_major(xs)                   # [G, K/128, ld]
    rows = xs.shape[1]
    view = store[:, :, :rows].transpose(1, 2)              # [G, M, K/128], column-major
    return view[0] if squeeze else view


def gemm_fp8_fp8_bf16_nt(lhs, rhs, out, stream=None) -> None:
    """out[m, n] = bf16(lhs @ rhs^T) with lhs = (a [M, K] FP8, scales [M, K/128] fp32,
    column-major) and rhs = (b [N, K] FP8, scales [N/128, K/128] fp32)."""
    (a, sa), (b, sb) = lhs, rhs
    dg_gemm_fp8_nt(a, _lhs_scales_mn_major(sa, "lhs"), b, sb, out, stream)


def m_grouped_gemm_fp8_fp8_bf16_nt_contiguous(lhs, rhs, out, m_indices, stream=None) -> None:
    """Contiguous layout: lhs = (a [M_total, K], scales [M_total, K/128] column-major),
    rhs = (b [G, N, K], scales [G, N/128, K/128]), m_indices [M_total] (group or -1)."""
    (a, sa), (b, sb) = lhs, rhs
    dg_m_grouped_gemm_fp8_contiguous(a, _lhs_scales_mn_major(sa, "lhs"), b, sb, out, m_indices, stream)


def m_grouped_gemm_fp8_fp8_bf16_nt_masked(lhs, rhs, out, masked_m, stream=None) -> None:
    """Masked layout: lhs = (a [G, max_m, K], scales [G, max_m, K/128], each group
    column-major), rhs = (b [G, N, K], scales [G, N/128, K/128]), masked_m [G] on the GPU."""
    import torch
    (a, sa), (b, sb) = lhs, rhs
    mn = _lhs_scales_mn_major(sa, "lhs")                   # [G, K/128, max_m] view, stride (., ld, 1)
    g, kb, max_m = mn.shape
    ld = mn.stride(1)
    if ld < max_m or mn.stride(0) != kb * ld:
        raise ValueError("lhs scales: groups must be stacked as [G][K/128][ld] (get_col_major_tma_aligned_tensor)")
    need = (mn.storage_offset() + g * kb * ld) * mn.element_size()
    if mn.untyped_storage().nbytes() < need:
        raise ValueError("lhs scales: the storage does not hold the padded leading dimension")
    full = torch.as_strided(mn, (g, kb, ld), (kb * ld, ld, 1))
    dg_m_grouped_gemm_fp8_masked(a, full, b, sb, out, masked_m, stream)


# ---- tuning and introspection hooks (dg_tuning.h: outside the library's contract)
def dg_set_kernel_config(config_id: int) -> None:
    """Pin a kernel configuration id for its layout (-1: automatic planning again)."""
    _check(load_library().dg_set_kernel_config(int(config_id)), "dg_set_kernel_config")


def dg_kernel_config_info() -> list:
    """All compiled kernel configurations as dicts (id, layout, block_m, block_n, waves,
    all_formats: whether E5M2 operands run in it, shape_specialised: whether it has
    instances compiled for fixed N and K, k_groups: 2 where two wave groups each sum
    every other K block and the sums are added at the end, else 1)."""
    out, res, i = (ctypes.c_int * 8)(), [], 0
    while load_library().dg_kernel_config_info(i, out) == DG_OK:
        res.append(dict(zip(("id", "layout", "block_m", "block_n", "waves", "all_formats", "shape_specialised",
                             "k_groups"), list(out))))
        i += 1
    return res


def dg_plan_tiles(m: int, n: int, num_units: int, block_ms, block_ns, eff=None, blocks_per_unit: int = 1):
    """Host-only planner; returns (index, block_m, block_n, tiles, waves)."""
    bm = (ctypes.c_int * len(block_ms))(*block_ms)
    bn = (ctypes.c_int * len(block_ns))(*block_ns)
    e = None if eff is None else (ctypes.c_double * len(eff))(*eff)
    out = (ctypes.c_int * 4)()
    r = load_library().dg_plan_tiles(m, n, num_units, blocks_per_unit, bm, len(block_ms), bn, len(block_ns),
                                     e, out)
    if r < 0:
        raise DGError(r, "dg_plan_tiles")
    return r, out[0], out[1], out[2], out[3]


def dg_describe_launch(layout: int, m: int, n: int, k: int, num_groups: int = 1, num_cus: int = 0) -> dict:
    """The launch a call of these sizes would make (layout 0 dense, 1 contiguous, 2 masked)."""
    out = (ctypes.c_int * 8)()
    r = load_library().dg_describe_launch(layout, m, n, k, num_groups, num_cus, out)
    _check(r, "dg_describe_launch")
    keys = ("block_m", "block_n", "waves_per_workgroup", "tiles", "grid", "config_id", "group_m",
            "k_blocks_specialised")
    return dict(zip(keys, list(out)))


__all__ = [
    "DGError", "load_library", "status_string", "dg_status_string",
    "dg_get_m_alignment", "dg_set_num_cus", "dg_get_num_cus",
    "dg_gemm_fp8_nt", "dg_gemm_fp8_nt_fmt", "DG_FMT_E4M3", "DG_FMT_E5M2", "dg_m_grouped_gemm_fp8_contiguous", "dg_m_grouped_gemm_fp8_masked",
    "dg_m_grouped_gemm_fp8_contiguous_fmt", "dg_m_grouped_gemm_fp8_masked_fmt",
    "dg_quantize_fp8_1x128", "dg_quantize_fp8_128x128", "dg_quantize_fp8_1x128_fmt",
    "dg_quantize_fp8_128x128_fmt", "dg_get_aligned_ld_sa", "dg_transform_sa_mn_major",
    "dg_check_contiguous_layout", "dg_plan_tiles",
    "dg_set_kernel_config", "dg_kernel_config_info", "dg_describe_launch",
    "gemm_fp8_fp8_bf16_nt", "m_grouped_gemm_fp8_fp8_bf16_nt_contiguous", "m_grouped_gemm_fp8_fp8_bf16_nt_masked",
    "set_num_sms", "get_num_sms", "get_m_alignment_for_contiguous_layout", "get_tma_aligned_size",
    "get_col_major_tma_aligned_tensor",
]
