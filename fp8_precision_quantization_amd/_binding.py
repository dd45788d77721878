"""ctypes binding of libmxcast (include/mxcast.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch (device memory is the only thing torch provides here),
and every call goes to the C ABI on torch's current HIP stream.  There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmxcast.so")

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_GROUPS, MX_ERR_HIP, MX_ERR_ALIGN, MX_ERR_WORKSPACE = range(7)
MX_BLOCK = 32
MX_MAX_GROUPS = 1024

_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

SIGNATURES = {
    "mx_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "mx_cast_dim0_dim1": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mx_cast_dim1_3d": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mx_cast_dim0_dim1_blocked": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mx_cast_dim1_3d_blocked": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mx_cast_dim0_dim1_mgrouped": ([_vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mx_cast_dim0_dim1_grouped_blocked": ([_vp, _i64, _i64, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
                                          ctypes.c_int),
    "mx_quantize_fp8_rowwise": ([_vp, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mx_tensorwise_workspace_bytes": ([_i64], _i64),
    "mx_quantize_fp8_tensorwise": ([_vp, _i64, _vp, _vp, _vp, _i64, _vp], ctypes.c_int),
    "mx_quantize_fp8_tensorwise_noalloc": ([_vp, _i64, _vp, _vp, _vp], ctypes.c_int),
    "mx_gemm_mxfp8": ([_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _vp], ctypes.c_int),
    "mx_grouped_gemm_mxfp8": ([_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp], ctypes.c_int),
    "mx_kgrouped_gemm_mxfp8": ([_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _vp, _i32, _vp], ctypes.c_int),
    "mx_blocked_bytes": ([_i64, _i64, _i64], _i64),
    "mx_scales_to_blocked": ([_vp, _i64, _i64, _i64, _vp, _vp], ctypes.c_int),
    "mx_blocked_grouped_bytes": ([_i64, _i64, _i32, _i32], _i64),
    "mx_scales_to_blocked_grouped": ([_vp, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _vp],
                                     ctypes.c_int),
}


class MxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libmxcast.so is missing at %s; build it with "
                    "`python -m fp8_precision_quantization_amd.build`" % LIB_PATH)
            handle = ctypes.CDLL(LIB_PATH)
            for name, (args, res) in SIGNATURES.items():
                f = getattr(handle, name)
                f.argtypes = args
                f.restype = res
            _lib = handle
        return _lib


def status_string(status: int) -> str:
    return lib().mx_status_string(status).decode()


def _check(status: int, where: str):
    if status != MX_OK:
        raise MxError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _as_u8(t):
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def _out(t, shape, device, name):
    if t is None:
        return torch.empty(shape, dtype=torch.uint8, device=device)
    t = _as_u8(t)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError("%s must be a contiguous %s tensor on %s" % (name, tuple(shape), device))
    return t


def _bf16_input(x, ndim, name):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if x.dtype != torch.bfloat16:
        raise ValueError("%s must be bfloat16, got %s" % (name, x.dtype))
    if x.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _pad(v, m):
    return (v + m - 1) // m * m


def _views(q, s, raw):
    if raw:
        return q, s
    return q.view(torch.float8_e4m3fn), s.view(torch.float8_e8m0fnu)


def mx_cast_dim0_dim1(x, dim0: bool = True, dim1: bool = True, out=None, raw: bool = False):
    """bf16 (R, C) -> (q_row (R, C), s_row (R, C/32), q_col (C, R), s_col (C, R/32)).

    q_col is the col-major cast stored as a row-major (C, R) array.  A
    direction turned off returns None for its pair.  `out` may hold
    preallocated uint8 outputs in the same order.  Results are e4m3 / e8m0
    views unless raw=True (uint8)."""
    _bf16_input(x, 2, "x")
    rows, cols = x.shape
    o = out if out is not None else (None, None, None, None)
    q0 = _out(o[0], (rows, cols), x.device, "q_row") if dim0 else None
    s0 = _out(o[1], (rows, cols // MX_BLOCK), x.device, "s_row") if dim0 else None
    q1 = _out(o[2], (cols, rows), x.device, "q_col") if dim1 else None
    s1 = _out(o[3], (cols, rows // MX_BLOCK), x.device, "s_col") if dim1 else None
    _check(lib().mx_cast_dim0_dim1(_ptr(x), rows, cols, _ptr(q0), _ptr(s0), _ptr(q1), _ptr(s1),
                                   _stream(x.device)), "mx_cast_dim0_dim1")
    r0 = _views(q0, s0, raw) if dim0 else (None, None)
    r1 = _views(q1, s1, raw) if dim1 else (None, None)
    return r0[0], r0[1], r1[0], r1[1]


def mx_cast_dim1_3d(w, out=None, raw: bool = False):
    """bf16 (E, N, K) -> (q (E, K, N), s (E, K, N/32)), per-expert dim1 cast."""
    _bf16_input(w, 3, "w")
    e, n, k = w.shape
    o = out if out is not None else (None, None)
    q = _out(o[0], (e, k, n), w.device, "q")
    s = _out(o[1], (e, k, n // MX_BLOCK), w.device, "s")
    _check(lib().mx_cast_dim1_3d(_ptr(w), e, n, k, _ptr(q), _ptr(s), _stream(w.device)),
           "mx_cast_dim1_3d")
    return _views(q, s, raw)


def mx_cast_dim0_dim1_blocked(x, dim0: bool = True, dim1: bool = True, out=None, raw: bool = False):
    """As mx_cast_dim0_dim1, with both scale sets written directly in the
    128x4 blocked layout: s_row as (ceil128(R), ceil4(C/32)) and s_col as
    (ceil128(C), ceil4(R/32)), padding 0."""
    _bf16_input(x, 2, "x")
    rows, cols = x.shape
    o = out if out is not None else (None, None, None, None)
    q0 = _out(o[0], (rows, cols), x.device, "q_row") if dim0 else None
    s0 = _out(o[1], (_pad(rows, 128), _pad(cols // MX_BLOCK, 4)), x.device, "s_row_blocked") if dim0 else None
    q1 = _out(o[2], (cols, rows), x.device, "q_col") if dim1 else None
    s1 = _out(o[3], (_pad(cols, 128), _pad(rows // MX_BLOCK, 4)), x.device, "s_col_blocked") if dim1 else None
    _check(lib().mx_cast_dim0_dim1_blocked(_ptr(x), rows, cols, _ptr(q0), _ptr(s0), _ptr(q1), _ptr(s1),
                                           _stream(x.device)), "mx_cast_dim0_dim1_blocked")
    r0 = _views(q0, s0, raw) if dim0 else (None, None)
    r1 = _views(q1, s1, raw) if dim1 else (None, None)
    return r0[0], r0[1], r1[0], r1[1]


def _offsets(offs, name="group_end_offsets"):
    if not (isinstance(offs, torch.Tensor) and offs.is_cuda and offs.dtype == torch.int32
            and offs.dim() == 1 and offs.is_contiguous()):
        raise ValueError("%s must be a contiguous int32 CUDA tensor" % name)
    return offs


def mx_cast_dim0_dim1_mgrouped(x, group_end_offsets, dim1: bool = True, out=None, out_group_starts=None,
                               raw: bool = False):
    """MoE activations grouped along M: as mx_cast_dim0_dim1, with the row
    scales written directly in the M-grouped blocked layout ((R + 128 G,
    ceil4(C/32)), what mx_scales_to_blocked_grouped(s_row, offsets, 0)
    gives).  Returns (q_row, s_row_grouped, starts, q_col, s_col); starts is
    int64 [G + 1] on the device; q_col / s_col are None when dim1 is False."""
    _bf16_input(x, 2, "x")
    offs = _offsets(group_end_offsets)
    rows, cols = x.shape
    g = offs.numel()
    o = out if out is not None else (None, None, None, None)
    q0 = _out(o[0], (rows, cols), x.device, "q_row")
    s0 = _out(o[1], (rows + 128 * g, _pad(cols // MX_BLOCK, 4)), x.device, "s_row_grouped")
    q1 = _out(o[2], (cols, rows), x.device, "q_col") if dim1 else None
    s1 = _out(o[3], (cols, rows // MX_BLOCK), x.device, "s_col") if dim1 else None
    if out_group_starts is None:
        starts = torch.empty(g + 1, dtype=torch.int64, device=x.device)
    else:
        starts = out_group_starts
        if starts.dtype != torch.int64 or starts.numel() != g + 1 or not starts.is_contiguous():
            raise ValueError("out_group_starts must be a contiguous int64 tensor of G + 1")
    _check(lib().mx_cast_dim0_dim1_mgrouped(_ptr(x), rows, cols, _ptr(offs), g, _ptr(q0), _ptr(s0),
                                            _ptr(starts), _ptr(q1), _ptr(s1), _stream(x.device)),
           "mx_cast_dim0_dim1_mgrouped")
    r0 = _views(q0, s0, raw)
    r1 = _views(q1, s1, raw) if dim1 else (None, None)
    return r0[0], r0[1], starts, r1[0], r1[1]


def _starts_out(t, g, dev, name):
    if t is None:
        return torch.empty(g + 1, dtype=torch.int64, device=dev)
    if t.dtype != torch.int64 or t.numel() != g + 1 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous int64 tensor of G + 1" % name)
    return t


def mx_cast_dim0_dim1_grouped_blocked(x, group_end_offsets, out=None, out_row_starts=None, out_col_starts=None,
                                      raw: bool = False):
    """MoE activations grouped along M, both scale sets in grouped blocked
    layouts: the row scales M-grouped ((R + 128 G, ceil4(C/32)), as
    mx_cast_dim0_dim1_mgrouped) and the column scales K-grouped along their
    32-row blocks ((ceil128(C), ceil4(R/32) + 4 G), what
    mx_scales_to_blocked_grouped(s_col, offsets // 32, 1) gives).  Returns
    (q_row, s_row_grouped, row_starts, q_col, s_col_grouped, col_starts)."""
    _bf16_input(x, 2, "x")
    offs = _offsets(group_end_offsets)
    rows, cols = x.shape
    g = offs.numel()
    o = out if out is not None else (None, None, None, None)
    q0 = _out(o[0], (rows, cols), x.device, "q_row")
    s0 = _out(o[1], (rows + 128 * g, _pad(cols // MX_BLOCK, 4)), x.device, "s_row_grouped")
    q1 = _out(o[2], (cols, rows), x.device, "q_col")
    s1 = _out(o[3], (_pad(cols, 128), _pad(rows // MX_BLOCK, 4) + 4 * g), x.device, "s_col_grouped")
    rs = _starts_out(out_row_starts, g, x.device, "out_row_starts")
    cs = _starts_out(out_col_starts, g, x.device, "out_col_starts")
    _check(lib().mx_cast_dim0_dim1_grouped_blocked(_ptr(x), rows, cols, _ptr(offs), g, _ptr(q0), _ptr(s0),
                                                   _ptr(rs), _ptr(q1), _ptr(s1), _ptr(cs), _stream(x.device)),
           "mx_cast_dim0_dim1_grouped_blocked")
    r0 = _views(q0, s0, raw)
    r1 = _views(q1, s1, raw)
    return r0[0], r0[1], rs, r1[0], r1[1], cs


def mx_cast_dim1_3d_blocked(w, out=None, raw: bool = False):
    """bf16 (E, N, K) -> (q (E, K, N), s (E, ceil128(K), ceil4(N/32))): the
    per-expert dim1 cast with each expert's scales in the blocked layout.
    N must be a multiple of 128."""
    _bf16_input(w, 3, "w")
    e, n, k = w.shape
    o = out if out is not None else (None, None)
    q = _out(o[0], (e, k, n), w.device, "q")
    s = _out(o[1], (e, _pad(k, 128), _pad(n // MX_BLOCK, 4)), w.device, "s_blocked")
    _check(lib().mx_cast_dim1_3d_blocked(_ptr(w), e, n, k, _ptr(q), _ptr(s), _stream(w.device)),
           "mx_cast_dim1_3d_blocked")
    return _views(q, s, raw)


def mx_quantize_fp8_rowwise(x, out=None, raw: bool = False):
    """bf16 (R, C) -> (q (R, C) e4m3fn, scale (R,) bf16): one scale per row,
    scale = amax / 448 (bf16), q = x / scale without saturation.  `out` may
    hold preallocated (uint8 (R, C), bf16 or int16 (R,)) outputs.  raw=True
    returns q as uint8 and the scale as its int16 bit patterns."""
    _bf16_input(x, 2, "x")
    rows, cols = x.shape
    o = out if out is not None else (None, None)
    q = _out(o[0], (rows, cols), x.device, "q")
    if o[1] is None:
        s = torch.empty(rows, dtype=torch.bfloat16, device=x.device)
    else:
        s = o[1]
        if (s.dtype not in (torch.bfloat16, torch.int16) or tuple(s.shape) != (rows,)
                or not s.is_contiguous() or s.device != x.device):
            raise ValueError("scale must be a contiguous bf16 or int16 (%d,) tensor on %s" % (rows, x.device))
    _check(lib().mx_quantize_fp8_rowwise(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(x.device)),
           "mx_quantize_fp8_rowwise")
    if raw:
        return q, s.view(torch.int16)
    return q.view(torch.float8_e4m3fn), s.view(torch.bfloat16)


def mx_tensorwise_workspace_bytes(n: int) -> int:
    return lib().mx_tensorwise_workspace_bytes(n)


def mx_quantize_fp8_tensorwise(x, out=None, workspace=None, raw: bool = False):
    """bf16 tensor of any shape -> (q same shape e4m3fn, scale bf16 (1,)): one
    scale for the whole tensor, scale = amax / 448 (bf16), q = x / scale
    without saturation.  `out` may hold preallocated (uint8 q, bf16 or int16
    (1,) scale); `workspace` a uint8 device tensor of at least
    mx_tensorwise_workspace_bytes(numel) bytes (allocated here if None)."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x must be a bfloat16 CUDA (HIP) tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    n = x.numel()
    o = out if out is not None else (None, None)
    q = _out(o[0], tuple(x.shape), x.device, "q")
    if o[1] is None:
        s = torch.empty(1, dtype=torch.bfloat16, device=x.device)
    else:
        s = o[1]
        if (s.dtype not in (torch.bfloat16, torch.int16) or s.numel() != 1 or not s.is_contiguous()
                or s.device != x.device):
            raise ValueError("scale must be a one-element bf16 or int16 tensor on %s" % x.device)
    need = max(lib().mx_tensorwise_workspace_bytes(n), 0)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    elif not (workspace.is_cuda and workspace.is_contiguous() and workspace.device == x.device):
        raise ValueError("workspace must be a contiguous tensor on %s" % x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().mx_quantize_fp8_tensorwise(_ptr(x), n, _ptr(q), _ptr(s), _ptr(workspace), ws_bytes,
                                            _stream(x.device)), "mx_quantize_fp8_tensorwise")
    if raw:
        return q, s.view(torch.int16)
    return q.view(torch.float8_e4m3fn), s.view(torch.bfloat16)


def mx_quantize_fp8_tensorwise_noalloc(x, out=None, raw: bool = False):
    """mx_quantize_fp8_tensorwise with the block amaxes in the library's
    static per-GPU scratch instead of a workspace (nothing is allocated when
    `out` is given).  Calls that overlap on one GPU race."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype != torch.bfloat16:
        raise ValueError("x must be a bfloat16 CUDA (HIP) tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    o = out if out is not None else (None, None)
    q = _out(o[0], tuple(x.shape), x.device, "q")
    if o[1] is None:
        s = torch.empty(1, dtype=torch.bfloat16, device=x.device)
    else:
        s = o[1]
        if (s.dtype not in (torch.bfloat16, torch.int16) or s.numel() != 1 or not s.is_contiguous()
                or s.device != x.device):
            raise ValueError("scale must be a one-element bf16 or int16 tensor on %s" % x.device)
    _check(lib().mx_quantize_fp8_tensorwise_noalloc(_ptr(x), x.numel(), _ptr(q), _ptr(s), _stream(x.device)),
           "mx_quantize_fp8_tensorwise_noalloc")
    if raw:
        return q, s.view(torch.int16)
    return q.view(torch.float8_e4m3fn), s.view(torch.bfloat16)


def _mx_operand(q, s, rows, k, nbytes, name):
    """Codes (..., rows, k) and their scales as blocked-layout bytes (any
    contiguous u8 tensor of nbytes elements)."""
    q = _scale_input(q, name + " codes")
    s = _scale_input(s, name + " scales")
    if tuple(q.shape[-2:]) != (rows, k):
        raise ValueError("%s: codes (%d, %d) expected" % (name, rows, k))
    if s.numel() != nbytes:
        raise ValueError("%s: %d bytes of blocked scales expected, got %d" % (name, nbytes, s.numel()))
    return q, s


def _gemm_out(out, shape, out_dtype, device):
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        return torch.empty(shape, dtype=out_dtype, device=device)
    if out.dtype != out_dtype or tuple(out.shape) != tuple(shape) or not out.is_contiguous() or out.device != device:
        raise ValueError("out must be a contiguous %s %s tensor on %s" % (out_dtype, tuple(shape), device))
    return out


def mx_gemm_mxfp8(qa, sa, qb, sb, out_dtype=torch.bfloat16, out=None):
    """C (M, N) = A @ B^T for MX operands: qa (M, K) e4m3 codes with sa the
    blocked layout of its (M, K/32) e8m0 scales, qb (N, K) with sb likewise
    -- the dim0 cast's outputs in its blocked-scale form."""
    m, k = qa.shape
    n = qb.shape[0]
    qa, sa = _mx_operand(qa, sa, m, k, mx_blocked_bytes(1, m, k // MX_BLOCK), "A")
    qb, sb = _mx_operand(qb, sb, n, k, mx_blocked_bytes(1, n, k // MX_BLOCK), "B")
    c = _gemm_out(out, (m, n), out_dtype, qa.device)
    _check(lib().mx_gemm_mxfp8(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), m, n, k, _ptr(c),
                               int(out_dtype == torch.bfloat16), _stream(qa.device)), "mx_gemm_mxfp8")
    return c


def mx_grouped_gemm_mxfp8(qa, sa, qb, sb, group_end_offsets, out_dtype=torch.bfloat16, out=None):
    """Grouped along M: rows of group g of A times group g's weights.  sa is
    the M-grouped blocked layout of A's scales (as mx_cast_dim0_dim1_mgrouped
    writes it), qb (G, N, K) the weights' codes and sb the G blocked layouts
    of their (N, K/32) scales one after another; offsets int32 [G] on the
    device.  Rows past the last end are left as they were in `out`."""
    m, k = qa.shape
    g, n, _ = qb.shape
    offs = _offsets(group_end_offsets)
    if offs.numel() != g:
        raise ValueError("one offset per group of B")
    qa, sa = _mx_operand(qa, sa, m, k, mx_blocked_grouped_bytes(m, k // MX_BLOCK, g, 0), "A")
    qb, sb = _mx_operand(qb, sb, n, k, mx_blocked_bytes(g, n, k // MX_BLOCK), "B")
    c = _gemm_out(out, (m, n), out_dtype, qa.device)
    _check(lib().mx_grouped_gemm_mxfp8(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _ptr(offs), g, m, n, k, _ptr(c),
                                       int(out_dtype == torch.bfloat16), _stream(qa.device)),
           "mx_grouped_gemm_mxfp8")
    return c


def mx_kgrouped_gemm_mxfp8(qa, sa, qb, sb, group_end_offsets, out_dtype=torch.bfloat16, out=None):
    """Grouped along K (the weight-gradient GEMM of MoE training): for each
    group g, C_g = A_g @ B_g^T over the group's K range (its 32-blocks
    [lo // 32, hi // 32) of the token offsets).  qa (M, K) and qb (N, K) are
    col-major casts (q_col), sa / sb their scales in the K-grouped blocked
    layout (as mx_cast_dim0_dim1_grouped_blocked writes s_col_grouped).
    Returns C (G, M, N)."""
    m, k = qa.shape
    n = qb.shape[0]
    offs = _offsets(group_end_offsets)
    g = offs.numel()
    qa, sa = _mx_operand(qa, sa, m, k, mx_blocked_grouped_bytes(m, k // MX_BLOCK, g, 1), "A")
    qb, sb = _mx_operand(qb, sb, n, k, mx_blocked_grouped_bytes(n, k // MX_BLOCK, g, 1), "B")
    c = _gemm_out(out, (g, m, n), out_dtype, qa.device)
    _check(lib().mx_kgrouped_gemm_mxfp8(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), _ptr(offs), g, m, n, k, _ptr(c),
                                        int(out_dtype == torch.bfloat16), _stream(qa.device)),
           "mx_kgrouped_gemm_mxfp8")
    return c


def mx_blocked_bytes(batch: int, rows: int, cols: int) -> int:
    return lib().mx_blocked_bytes(batch, rows, cols)


def mx_blocked_grouped_bytes(rows: int, cols: int, num_groups: int, group_axis: int) -> int:
    return lib().mx_blocked_grouped_bytes(rows, cols, num_groups, group_axis)


def _scale_input(s, name="scales"):
    if not isinstance(s, torch.Tensor) or not s.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    s = _as_u8(s)
    if not s.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return s


def mx_scales_to_blocked(s, out=None, raw: bool = False):
    """e8m0 (R, C) or (B, R, C) -> blocked layout, shaped (ceil128(R), ceil4(C))
    or (B, ceil128(R), ceil4(C)); every byte written."""
    s = _scale_input(s)
    if s.dim() == 2:
        batch, (rows, cols) = 1, s.shape
        shape = (_pad(rows, 128), _pad(cols, 4))
    elif s.dim() == 3:
        batch, rows, cols = s.shape
        shape = (batch, _pad(rows, 128), _pad(cols, 4))
    else:
        raise ValueError("scales must be 2D or 3D")
    o = _out(out, shape, s.device, "out")
    _check(lib().mx_scales_to_blocked(_ptr(s), batch, rows, cols, _ptr(o), _stream(s.device)),
           "mx_scales_to_blocked")
    return o if raw else o.view(torch.float8_e8m0fnu)


def mx_scales_to_blocked_grouped(s, group_end_offsets, group_axis: int, out=None,
                                 out_group_starts=None, raw: bool = False):
    """Grouped blocked layout with device-side END offsets (int32 [G]).

    Returns (out, starts): out is (R + 128 G, ceil4(C)) for group_axis 0 and
    (ceil128(R), ceil4(C) + 4 G) for group_axis 1; starts is int64 [G + 1] on
    the device (padded start of each group, then the total)."""
    s = _scale_input(s)
    if s.dim() != 2:
        raise ValueError("scales must be 2D")
    offs = group_end_offsets
    if not (isinstance(offs, torch.Tensor) and offs.is_cuda and offs.dtype == torch.int32
            and offs.dim() == 1 and offs.is_contiguous()):
        raise ValueError("group_end_offsets must be a contiguous int32 CUDA tensor")
    rows, cols = s.shape
    g = offs.numel()
    if group_axis == 0:
        shape = (rows + 128 * g, _pad(cols, 4))
    elif group_axis == 1:
        shape = (_pad(rows, 128), _pad(cols, 4) + 4 * g)
    else:
        raise ValueError("group_axis must be 0 or 1")
    o = _out(out, shape, s.device, "out")
    if out_group_starts is None:
        starts = torch.empty(g + 1, dtype=torch.int64, device=s.device)
    else:
        starts = out_group_starts
        if starts.dtype != torch.int64 or starts.numel() != g + 1 or not starts.is_contiguous():
            raise ValueError("out_group_starts must be a contiguous int64 tensor of G + 1")
    _check(lib().mx_scales_to_blocked_grouped(_ptr(s), rows, cols, _ptr(offs), g, group_axis,
                                              _ptr(o), _ptr(starts), _stream(s.device)),
           "mx_scales_to_blocked_grouped")
    return (o if raw else o.view(torch.float8_e8m0fnu)), starts
