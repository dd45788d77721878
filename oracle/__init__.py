"""CPU oracle for the bf16 -> MXFP8 cast, the 128x4 blocked scale layout and
the row-wise and tensor-wise fp8 casts.

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or runs
anything here; only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` do.  The arithmetic lives in ``mxoracle.c`` (plain C99,
fp64, one block at a time); this module compiles it with gcc and marshals
numpy arrays through ctypes.  Every function takes and returns host numpy
arrays: bf16 data as its uint16 bit patterns, fp8/e8m0 results as uint8.

Each function's rule and its source passage are stated in ``mxoracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libmxoracle.so")
_lock = threading.Lock()
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile mxoracle.c into _build/libmxoracle.so (gcc, -O2, OpenMP)."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    if (not force and os.path.exists(_LIB)
            and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC)):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-Wall", "-Werror", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build())
        lib.mxo_bf16_value.argtypes = [ctypes.c_uint16]
        lib.mxo_bf16_value.restype = ctypes.c_double
        lib.mxo_e4m3_value.argtypes = [ctypes.c_int]
        lib.mxo_e4m3_value.restype = ctypes.c_double
        lib.mxo_e8m0_value.argtypes = [ctypes.c_int]
        lib.mxo_e8m0_value.restype = ctypes.c_double
        lib.mxo_scale_byte.argtypes = [ctypes.c_double]
        lib.mxo_scale_byte.restype = ctypes.c_int
        lib.mxo_quantize_element.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.mxo_quantize_element.restype = ctypes.c_int
        lib.mxo_quantize_elements.argtypes = [_u16p, _i64, ctypes.c_int, _u8p]
        lib.mxo_quantize_elements.restype = None
        lib.mxo_quantize_block.argtypes = [_u16p, _u8p, _u8p]
        lib.mxo_quantize_block.restype = None
        for name in ("mxo_cast_dim0", "mxo_cast_dim1"):
            f = getattr(lib, name)
            f.argtypes = [_u16p, _i64, _i64, _u8p, _u8p]
            f.restype = ctypes.c_int
        lib.mxo_cast_dim1_3d.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _u8p]
        lib.mxo_cast_dim1_3d.restype = ctypes.c_int
        lib.mxo_blocked_size.argtypes = [_i64, _i64]
        lib.mxo_blocked_size.restype = _i64
        lib.mxo_to_blocked.argtypes = [_u8p, _i64, _i64, _u8p]
        lib.mxo_to_blocked.restype = ctypes.c_int
        lib.mxo_to_blocked_batched.argtypes = [_u8p, _i64, _i64, _i64, _u8p]
        lib.mxo_to_blocked_batched.restype = ctypes.c_int
        lib.mxo_blocked_grouped_size.argtypes = [_i64, _i64, ctypes.c_int32, ctypes.c_int32]
        lib.mxo_blocked_grouped_size.restype = _i64
        lib.mxo_to_blocked_grouped.argtypes = [_u8p, _i64, _i64, _i32p, ctypes.c_int32,
                                               ctypes.c_int32, _u8p, _i64, _i64p]
        lib.mxo_to_blocked_grouped.restype = ctypes.c_int
        lib.mxo_bf16_round.argtypes = [ctypes.c_float]
        lib.mxo_bf16_round.restype = ctypes.c_uint16
        lib.mxo_e4m3fn_from_f32.argtypes = [ctypes.c_float]
        lib.mxo_e4m3fn_from_f32.restype = ctypes.c_int
        lib.mxo_rowwise_scale.argtypes = [ctypes.c_double]
        lib.mxo_rowwise_scale.restype = ctypes.c_uint16
        lib.mxo_rowwise_element.argtypes = [ctypes.c_double, ctypes.c_uint16]
        lib.mxo_rowwise_element.restype = ctypes.c_int
        lib.mxo_rowwise_elements.argtypes = [_u16p, _i64, ctypes.c_uint16, _u8p]
        lib.mxo_rowwise_elements.restype = None
        lib.mxo_quantize_fp8_rowwise.argtypes = [_u16p, _i64, _i64, _u8p, _u16p]
        lib.mxo_quantize_fp8_rowwise.restype = ctypes.c_int
        lib.mxo_quantize_fp8_tensorwise.argtypes = [_u16p, _i64, _u8p, _u16p]
        lib.mxo_quantize_fp8_tensorwise.restype = ctypes.c_int
        _f64p = ctypes.POINTER(ctypes.c_double)
        lib.mxo_mx_gemm.argtypes = [_u8p, _u8p, _u8p, _u8p, _i64, _i64, _i64, _f64p, _f64p]
        lib.mxo_mx_gemm.restype = ctypes.c_int
        lib.mxo_mx_gemm_grouped.argtypes = [_u8p, _u8p, _u8p, _u8p, _i32p, ctypes.c_int32, _i64, _i64, _i64,
                                            _f64p, _f64p]
        lib.mxo_mx_gemm_grouped.restype = ctypes.c_int
        lib.mxo_num_threads.argtypes = []
        lib.mxo_num_threads.restype = ctypes.c_int
        lib.mxo_set_num_threads.argtypes = [ctypes.c_int]
        lib.mxo_set_num_threads.restype = None
        _lib = lib
        return lib


def _ptr(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 data is passed as uint16 bit patterns, got %s" % x.dtype)
    return x


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (code %d)" % (what, rc))


# ---------------------------------------------------------------- formats
def bf16_value(bits: int) -> float:
    return _load().mxo_bf16_value(bits)


def e4m3_value(code: int) -> float:
    """Value of an e4m3fn magnitude code 0x00..0x7E."""
    return _load().mxo_e4m3_value(code)


def e8m0_value(byte: int) -> float:
    return _load().mxo_e8m0_value(byte)


# ---------------------------------------------------------------- MX rule
def scale_byte(amax: float) -> int:
    """e8m0 byte of a block with this amax (>= 0 or NaN)."""
    return _load().mxo_scale_byte(float(amax))


def quantize_element(x: float, s: int) -> int:
    """e4m3 byte of the value x under e8m0 scale byte s."""
    return _load().mxo_quantize_element(float(x), int(s))


def quantize_elements(bits: np.ndarray, s: int) -> np.ndarray:
    """Element rule over bf16 bit patterns, one scale byte for all."""
    x = _bits(bits).reshape(-1)
    q = np.empty(x.shape, np.uint8)
    _load().mxo_quantize_elements(_ptr(x, _u16p), x.size, int(s), _ptr(q, _u8p))
    return q.reshape(bits.shape)


def quantize_block(bits32: np.ndarray):
    """One 32-element block -> (32 e4m3 bytes, e8m0 byte)."""
    x = _bits(bits32).reshape(-1)
    if x.size != 32:
        raise ValueError("a block has 32 elements")
    q = np.empty(32, np.uint8)
    s = np.empty(1, np.uint8)
    _load().mxo_quantize_block(_ptr(x, _u16p), _ptr(q, _u8p), _ptr(s, _u8p))
    return q, int(s[0])


# ---------------------------------------------------------------- casts
def cast_dim0(bits: np.ndarray):
    """(R, C) bf16 bits -> q (R, C) u8, s (R, C/32) u8."""
    x = _bits(bits)
    r, c = x.shape
    q = np.empty((r, c), np.uint8)
    s = np.empty((r, c // 32), np.uint8)
    _check(_load().mxo_cast_dim0(_ptr(x, _u16p), r, c, _ptr(q, _u8p), _ptr(s, _u8p)), "cast_dim0")
    return q, s


def cast_dim1(bits: np.ndarray):
    """(R, C) bf16 bits -> q (C, R) u8 (col-major of (R, C)), s (C, R/32) u8."""
    x = _bits(bits)
    r, c = x.shape
    q = np.empty((c, r), np.uint8)
    s = np.empty((c, r // 32), np.uint8)
    _check(_load().mxo_cast_dim1(_ptr(x, _u16p), r, c, _ptr(q, _u8p), _ptr(s, _u8p)), "cast_dim1")
    return q, s


def cast_dim1_3d(bits: np.ndarray):
    """(E, N, K) bf16 bits -> q (E, K, N) u8, s (E, K, N/32) u8."""
    w = _bits(bits)
    e, n, k = w.shape
    q = np.empty((e, k, n), np.uint8)
    s = np.empty((e, k, n // 32), np.uint8)
    _check(_load().mxo_cast_dim1_3d(_ptr(w, _u16p), e, n, k, _ptr(q, _u8p), _ptr(s, _u8p)),
           "cast_dim1_3d")
    return q, s


# ---------------------------------------------------------------- row-wise fp8
def bf16_round(f: float) -> int:
    """float32 value -> bf16 bits, nearest-even (NaN -> 0x7FC0)."""
    return int(_load().mxo_bf16_round(float(f)))


def e4m3fn_from_f32(f: float) -> int:
    """float32 value -> e4m3fn byte, nearest-even, no saturation (sign kept)."""
    return int(_load().mxo_e4m3fn_from_f32(float(f)))


def rowwise_scale(amax: float) -> int:
    """bf16 bits of the row scale for a row amax (a bf16 value or NaN)."""
    return int(_load().mxo_rowwise_scale(float(amax)))


def rowwise_element(x: float, scale_bits: int) -> int:
    """e4m3fn byte of the bf16 value x under a row scale given as bf16 bits."""
    return int(_load().mxo_rowwise_element(float(x), int(scale_bits)))


def rowwise_elements(bits: np.ndarray, scale_bits: int) -> np.ndarray:
    """e4m3fn bytes of bf16 values under one scale given as bf16 bits."""
    x = _bits(bits).reshape(-1)
    q = np.empty(x.shape, np.uint8)
    _load().mxo_rowwise_elements(_ptr(x, _u16p), x.size, int(scale_bits), _ptr(q, _u8p))
    return q.reshape(bits.shape)


def quantize_fp8_rowwise(bits: np.ndarray):
    """(R, C) bf16 bits -> q (R, C) e4m3fn bytes, scale (R,) bf16 bits."""
    x = _bits(bits)
    r, c = x.shape
    q = np.empty((r, c), np.uint8)
    s = np.zeros(r, np.uint16)
    _check(_load().mxo_quantize_fp8_rowwise(_ptr(x, _u16p), r, c, _ptr(q, _u8p), _ptr(s, _u16p)),
           "quantize_fp8_rowwise")
    return q, s


def quantize_fp8_tensorwise(bits: np.ndarray):
    """bf16 bits of any shape -> (q same shape e4m3fn bytes, scale bf16 bits)."""
    x = _bits(bits)
    q = np.empty(x.shape, np.uint8)
    s = np.zeros(1, np.uint16)
    _check(_load().mxo_quantize_fp8_tensorwise(_ptr(x.reshape(-1), _u16p), x.size, _ptr(q.reshape(-1), _u8p),
                                               _ptr(s, _u16p)), "quantize_fp8_tensorwise")
    return q, int(s[0])


# ---------------------------------------------------------------- MX GEMM
def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def mx_gemm(qa, sa, qb, sb):
    """C (M, N) fp64 and sum |A B| (M, N) for MX operands: qa (M, K) / sa
    (M, K/32), qb (N, K) / sb (N, K/32), codes e4m3 and scales e8m0 as uint8."""
    qa, sa, qb, sb = _u8(qa), _u8(sa), _u8(qb), _u8(sb)
    m, k = qa.shape
    n = qb.shape[0]
    c = np.empty((m, n), np.float64)
    ab = np.empty((m, n), np.float64)
    _f64p = ctypes.POINTER(ctypes.c_double)
    _check(_load().mxo_mx_gemm(_ptr(qa, _u8p), _ptr(sa, _u8p), _ptr(qb, _u8p), _ptr(sb, _u8p), m, n, k,
                               _ptr(c, _f64p), _ptr(ab, _f64p)), "mx_gemm")
    return c, ab


def mx_gemm_grouped(qa, sa, qb, sb, ends):
    """Grouped along M: qb (G, N, K), sb (G, N, K/32), ends int32 [G].  Rows
    past the last (clamped) end are NaN in the result."""
    qa, sa, qb, sb = _u8(qa), _u8(sa), _u8(qb), _u8(sb)
    ends = np.ascontiguousarray(ends, dtype=np.int32)
    m, k = qa.shape
    g, n, _ = qb.shape
    c = np.full((m, n), np.nan)
    ab = np.full((m, n), np.nan)
    _f64p = ctypes.POINTER(ctypes.c_double)
    _check(_load().mxo_mx_gemm_grouped(_ptr(qa, _u8p), _ptr(sa, _u8p), _ptr(qb, _u8p), _ptr(sb, _u8p),
                                       _ptr(ends, _i32p), g, m, n, k, _ptr(c, _f64p), _ptr(ab, _f64p)),
           "mx_gemm_grouped")
    return c, ab


# ---------------------------------------------------------------- layouts
def blocked_size(rows: int, cols: int) -> int:
    return _load().mxo_blocked_size(rows, cols)


def to_blocked(s: np.ndarray) -> np.ndarray:
    """(R, C) or (B, R, C) u8 scales -> flat blocked bytes (per matrix, concatenated)."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    if s.ndim == 2:
        r, c = s.shape
        out = np.empty(blocked_size(r, c), np.uint8)
        _check(_load().mxo_to_blocked(_ptr(s, _u8p), r, c, _ptr(out, _u8p)), "to_blocked")
        return out
    b, r, c = s.shape
    out = np.empty(b * blocked_size(r, c), np.uint8)
    _check(_load().mxo_to_blocked_batched(_ptr(s, _u8p), b, r, c, _ptr(out, _u8p)),
           "to_blocked_batched")
    return out


def blocked_grouped_size(rows: int, cols: int, groups: int, axis: int) -> int:
    return _load().mxo_blocked_grouped_size(rows, cols, groups, axis)


def to_blocked_grouped(s: np.ndarray, ends: np.ndarray, axis: int):
    """Grouped blocked layout -> (flat output bytes, int64 padded starts [G+1])."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    ends = np.ascontiguousarray(ends, dtype=np.int32)
    r, c = s.shape
    g = ends.size
    nbytes = blocked_grouped_size(r, c, g, axis)
    if nbytes < 0:
        raise ValueError("bad grouped-layout arguments")
    out = np.empty(nbytes, np.uint8)
    starts = np.empty(g + 1, np.int64)
    _check(_load().mxo_to_blocked_grouped(_ptr(s, _u8p), r, c, _ptr(ends, _i32p), g, axis,
                                          _ptr(out, _u8p), nbytes, _ptr(starts, _i64p)),
           "to_blocked_grouped")
    return out, starts


def num_threads() -> int:
    return _load().mxo_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls (timing only; results do not depend on it)."""
    _load().mxo_set_num_threads(n)
