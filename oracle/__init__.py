"""Reference oracle (test infrastructure only).

Plain host implementation of what the FP8/FP16 GEMM path computes, in double
precision (oracle.c holds the arithmetic and its citations). Only the tests,
the package smoke check and the benchmark's CPU-baseline leg may import this
module; the product library never does, and shares no code with it.

This wrapper only marshals numpy arrays into the C functions.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_E4M3 = 0
FMT_F16 = 1
FMT_E5M2 = 2

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from .build import build_oracle
        build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_f16_decode.restype = ctypes.c_double
    lib.orc_f16_decode.argtypes = [ctypes.c_uint16]
    lib.orc_f16_round.restype = ctypes.c_uint16
    lib.orc_f16_round.argtypes = [ctypes.c_double]
    lib.orc_e5m2_decode.restype = ctypes.c_double
    lib.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e5m2_encode.restype = ctypes.c_uint8
    lib.orc_e5m2_encode.argtypes = [ctypes.c_double]
    for name in ("orc_e4m3_decode_n", "orc_e4m3_encode_n", "orc_e4m3_encode_f32bits",
                 "orc_e5m2_decode_n", "orc_e5m2_encode_n", "orc_e5m2_encode_f32bits",
                 "orc_f16_decode_n", "orc_f16_round_n", "orc_out_f16"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [_vp, _c_i64, _vp]
    lib.orc_amax.restype = ctypes.c_float
    lib.orc_amax.argtypes = [_vp, _c_i64]
    lib.orc_scale_from_amax.restype = ctypes.c_float
    lib.orc_scale_from_amax.argtypes = [ctypes.c_float]
    lib.orc_quantize.restype = None
    lib.orc_quantize.argtypes = [_vp, _c_i64, ctypes.c_float, _vp]
    lib.orc_scale.restype = ctypes.c_float
    lib.orc_scale.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.orc_quantize_fmt.restype = None
    lib.orc_quantize_fmt.argtypes = [_vp, _c_i64, ctypes.c_float, ctypes.c_int, _vp]
    lib.orc_gemm.restype = ctypes.c_int
    lib.orc_gemm.argtypes = [ctypes.c_int, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]
    lib.orc_gemm_mixed.restype = ctypes.c_int
    lib.orc_gemm_mixed.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i64,
                                   _vp, _vp]
    lib.orc_out_fp8.restype = None
    lib.orc_out_fp8.argtypes = [_vp, _c_i64, ctypes.c_double, ctypes.c_int, _vp]
    lib.orc_out_e4m3.restype = None
    lib.orc_out_e4m3.argtypes = [_vp, _c_i64, ctypes.c_double, _vp]
    lib.orc_amax_channel.restype = None
    lib.orc_amax_channel.argtypes = [_vp, _c_i64, _c_i64, ctypes.c_int, _vp]
    lib.orc_scale_n.restype = None
    lib.orc_scale_n.argtypes = [_vp, _c_i64, ctypes.c_int, ctypes.c_int, _vp]
    lib.orc_quantize_channel.restype = None
    lib.orc_quantize_channel.argtypes = [_vp, _c_i64, _c_i64, ctypes.c_int, _vp, ctypes.c_int, _vp]
    lib.orc_guard_scale.restype = ctypes.c_float
    lib.orc_guard_scale.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.orc_guard_to_f16.restype = None
    lib.orc_guard_to_f16.argtypes = [_vp, _c_i64, ctypes.c_float, _vp]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(values) -> np.ndarray:
    """E4M3 code of each real value (given as float64), RNE, saturating."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_f32bits(bits) -> np.ndarray:
    b = _c(bits, np.uint32)
    out = np.empty(b.shape, np.uint8)
    _load().orc_e4m3_encode_f32bits(_ptr(b), b.size, _ptr(out))
    return out


def e5m2_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().orc_e5m2_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e5m2_encode(values) -> np.ndarray:
    """E5M2 code of each real value (given as float64), RNE, saturating at 57344."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e5m2_encode_n(_ptr(v), v.size, _ptr(out))
    return out


def e5m2_encode_f32bits(bits) -> np.ndarray:
    b = _c(bits, np.uint32)
    out = np.empty(b.shape, np.uint8)
    _load().orc_e5m2_encode_f32bits(_ptr(b), b.size, _ptr(out))
    return out


def fp8_decode(codes, fmt) -> np.ndarray:
    return e5m2_decode(codes) if fmt == FMT_E5M2 else e4m3_decode(codes)


def f16_decode(bits) -> np.ndarray:
    h = _c(bits, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().orc_f16_decode_n(_ptr(h), h.size, _ptr(out))
    return out


def f16_round(values) -> np.ndarray:
    """binary16 bit patterns (uint16) of each float64 value, RNE."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_f16_round_n(_ptr(v), v.size, _ptr(out))
    return out


def amax(x) -> np.float32:
    a = _c(x, np.float32)
    return np.float32(_load().orc_amax(_ptr(a), a.size))


def scale_from_amax(a) -> np.float32:
    return np.float32(_load().orc_scale_from_amax(float(np.float32(a))))


def scale(a, fmt=FMT_E4M3, pow2=False) -> np.float32:
    """Per-tensor scale of amax a for an FP8 format: a / fmax in FP32 (1 when
    that is 0), or with pow2 the smallest power of two s with a / s <= fmax."""
    return np.float32(_load().orc_scale(float(np.float32(a)), int(fmt), 1 if pow2 else 0))


def quantize(x, s, fmt=FMT_E4M3) -> np.ndarray:
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint8)
    if fmt == FMT_E4M3:
        _load().orc_quantize(_ptr(a), a.size, float(np.float32(s)), _ptr(out))
    else:
        _load().orc_quantize_fmt(_ptr(a), a.size, float(np.float32(s)), int(fmt), _ptr(out))
    return out


def amax_channel(x, axis) -> np.ndarray:
    """max|x| per row (axis 0) or per column (axis 1) of a 2-D float32 array;
    NaN in a channel makes its value NaN."""
    a = _c(x, np.float32)
    rows, cols = a.shape
    out = np.empty(rows if axis == 0 else cols, np.float32)
    _load().orc_amax_channel(_ptr(a), rows, cols, int(axis), _ptr(out))
    return out


def scale_channel(a, fmt=FMT_E4M3, pow2=False) -> np.ndarray:
    """The per-tensor scale rule applied to each channel's amax."""
    v = _c(a, np.float32)
    out = np.empty(v.shape, np.float32)
    _load().orc_scale_n(_ptr(v), v.size, int(fmt), 1 if pow2 else 0, _ptr(out))
    return out


def quantize_channel(x, s, axis, fmt=FMT_E4M3) -> np.ndarray:
    """FP8 codes of x[i,j] / s[i] (axis 0) or x[i,j] / s[j] (axis 1)."""
    a = _c(x, np.float32)
    rows, cols = a.shape
    sv = _c(s, np.float32)
    if sv.shape != ((rows,) if axis == 0 else (cols,)):
        raise ValueError("one scale per channel")
    out = np.empty(a.shape, np.uint8)
    _load().orc_quantize_channel(_ptr(a), rows, cols, int(axis), _ptr(sv), int(fmt), _ptr(out))
    return out


def guard_scale(amax_a, amax_b) -> np.float32:
    """FP16 dynamic-range guard scale min(1, 65504 / (amax_a * amax_b))."""
    return np.float32(_load().orc_guard_scale(float(np.float32(amax_a)), float(np.float32(amax_b))))


def guard_to_f16(x, s) -> np.ndarray:
    """binary16 bits (uint16) of x * sqrt(s), each rounded to FP32 and then FP16."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_guard_to_f16(_ptr(a), a.size, float(np.float32(s)), _ptr(out))
    return out


def gemm(fmt, A, B, rows=None, fmt_b=None):
    """Unscaled reference product of row-major A[M,K] and B[K,N].

    A, B: uint8 FP8 codes (fmt=FMT_E4M3 or FMT_E5M2; B may use another FP8
    format given as fmt_b) or uint16 binary16 bits (FMT_F16).
    Returns (R, S), float64 [len(rows) or M, N]: R = sum_k a*b in ascending k,
    S = sum_k |a*b|. rows: optional list of row indices to compute.
    """
    fb = fmt if fmt_b is None else fmt_b
    if (fmt == FMT_F16) != (fb == FMT_F16):
        raise ValueError("FP16 pairs only with FP16")
    dt = np.uint16 if fmt == FMT_F16 else np.uint8
    A = _c(A, dt)
    B = _c(B, dt)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if rows is None:
        nrows, rp = M, None
    else:
        r = _c(rows, np.int64)
        if r.size and (r.min() < 0 or r.max() >= M):
            raise ValueError("row index out of range")
        nrows, rp = r.size, _ptr(r)
    R = np.empty((nrows, N), np.float64)
    S = np.empty((nrows, N), np.float64)
    if nrows and N:
        rc = _load().orc_gemm_mixed(fmt, fb, _ptr(A), _ptr(B), M, N, K, rp, nrows, _ptr(R), _ptr(S))
        if rc != 0:
            raise MemoryError("oracle gemm: out of memory")
    return R, S


def out_f16(V) -> np.ndarray:
    return f16_round(V)


def out_fp8(V, s_out, fmt) -> np.ndarray:
    v = _c(V, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_out_fp8(_ptr(v), v.size, float(s_out), int(fmt), _ptr(out))
    return out


def out_e4m3(V, s_out) -> np.ndarray:
    v = _c(V, np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_out_e4m3(_ptr(v), v.size, float(s_out), _ptr(out))
    return out
