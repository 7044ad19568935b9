"""Python binding of libgemm (include/libgemm.h): argument marshalling only.

Every step of the GEMM path runs in the HIP kernels of libgemm.so; this module
only turns torch tensors (device memory) and streams into the C-ABI's plain
pointers and sizes, and turns negative statuses into exceptions. It has no
fallback: if libgemm.so is not built, every call raises.

Functions keep the C names:
    gemm_f16(A, B, C, stream=None)
    gemm_fp8_scaled(A, B, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    gemm_fp8_fmt(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    quantize_fp8(x, scale, q=None, stream=None) -> q
    quantize_fp8_fmt(x, scale, fmt, q=None, stream=None) -> q
    amax_f32(x, amax=None, scale=None, stream=None) -> (amax, scale)
    amax_scale_f32(x, fmt, pow2, amax=None, scale=None, stream=None) -> (amax, scale)
    gemm_fp8_channel(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    quantize_fp8_channel(x, scale, axis, fmt, q=None, stream=None) -> q
    amax_scale_channel_f32(x, axis, fmt, pow2, amax=None, scale=None, stream=None) -> (amax, scale)
    gemm_fp8_splitk(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, workspace=None, stream=None, out_fmt=None)
    gemm_fp8_splitk_noalloc(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    gemm_f16_splitk(A, B, C, workspace=None, stream=None)
    splitk_plan(kind, out_dtype, M, N, K, fmt_a=0, fmt_b=0) -> (config, splits, workspace_bytes)
    gemm_f16_guarded(A, B, C, scale=None, workspace=None, stream=None) -> (C, scale)
    guarded_workspace_size(M, N, K) -> int
    select_config(kind, out_dtype, M, N, K) -> str   (host-only query)
    select_config_fmt(kind, out_dtype, M, N, K, fmt_a, fmt_b) -> str
  K-major B (Bt[N,K], the layout of a linear layer's weight):
    gemm_f16_bt(A, Bt, C, stream=None)
    gemm_fp8_scaled_bt(A, Bt, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    quantize_fp8_transposed(x, scale, q=None, stream=None) -> q[cols, rows]
    gemm_fp8_fmt_bt(A, fmt_a, Bt, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    quantize_fp8_transposed_fmt(x, scale, fmt, q=None, stream=None) -> q[cols, rows]
    pack_b_kmajor(B, Bt=None, stream=None) -> Bt[N, K]   (FP16 or FP8 codes)
    select_config_bt(kind, out_dtype, M, N, K) -> str
    gemm_fp8_splitk_bt(A, Bt, sA, sB, C, sOut=None, workspace=None, stream=None, out_fmt=None)
    gemm_f16_splitk_bt(A, Bt, C, workspace=None, stream=None)
    splitk_plan_bt(kind, out_dtype, M, N, K) -> (config, splits, workspace_bytes)
  Both FP8 operands in two launches (amax, scale and quantize of A and B):
    amax_quantize_fp8_pair(xa, xb, fmt=FMT_E4M3, pow2=False, amax=None, scale=None, qa=None, qb=None,
                           workspace=None, stream=None) -> (amax[2], scale[2], qa, qb)
    amax_quantize_fp8_pair_bt(xa, xb, fmt=FMT_E4M3, pow2=False, amax=None, scale=None, qa=None, qbt=None,
                              workspace=None, stream=None) -> (amax[2], scale[2], qa, qbt[N, K])
  Exact-accumulation FP8 (FP8 codes widened to FP16, FP16 matrix cores):
    gemm_fp8_exact(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    gemm_fp8_exact_bt(A, fmt_a, Bt, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None)
    select_config_exact(out_dtype, M, N, K, fmt_a=0, fmt_b=0, b_kmajor=0) -> str
The output dtype of a GEMM is taken from C: float32, float16, or 8-bit codes
(uint8 or torch.float8_e4m3fn: E4M3; torch.float8_e5m2, or uint8 with
out_fmt=FMT_E5M2: E5M2). FP8 operands are uint8 codes or torch float8 tensors.
"""
import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgemm.so")

OUT_F32 = 0
OUT_F16 = 1
OUT_E4M3 = 2
OUT_E5M2 = 3
FMT_E4M3 = 0
FMT_E5M2 = 1
KIND_F16 = 0
KIND_FP8 = 1
AXIS_ROW = 0
AXIS_COL = 1

GEMM_OK = 0
STATUS_NAMES = {
    0: "GEMM_OK", -1: "GEMM_ERR_NULL", -2: "GEMM_ERR_DIM", -3: "GEMM_ERR_DTYPE",
    -4: "GEMM_ERR_SCALE", -5: "GEMM_ERR_LAUNCH", -6: "GEMM_ERR_UNSUPPORTED",
    -7: "GEMM_ERR_DEVICE", -8: "GEMM_ERR_ALIAS", -9: "GEMM_ERR_WORKSPACE",
}

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    """The loaded libgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python __graft_entry__.py build, "
                           "or python precision_dense_gemm_03_amd/_build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.gemm_f16.restype = i32
    L.gemm_f16.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp]
    L.gemm_fp8_scaled.restype = i32
    L.gemm_fp8_scaled.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.quantize_fp8.restype = i32
    L.quantize_fp8.argtypes = [vp, i64, vp, vp, vp]
    L.amax_f32.restype = i32
    L.amax_f32.argtypes = [vp, i64, vp, vp, vp]
    L.gemm_status_str.restype = ctypes.c_char_p
    L.gemm_status_str.argtypes = [i32]
    L.gemm_select_config.restype = i32
    L.gemm_select_config.argtypes = [i32, i32, i64, i64, i64, ctypes.c_char_p, i32]
    L.gemm_fp8_fmt.restype = i32
    L.gemm_fp8_fmt.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.quantize_fp8_fmt.restype = i32
    L.quantize_fp8_fmt.argtypes = [vp, i64, vp, vp, i32, vp]
    L.amax_scale_f32.restype = i32
    L.amax_scale_f32.argtypes = [vp, i64, vp, vp, i32, i32, vp]
    L.gemm_fp8_channel.restype = i32
    L.gemm_fp8_channel.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.amax_scale_channel_f32.restype = i32
    L.amax_scale_channel_f32.argtypes = [vp, i64, i64, i32, vp, vp, i32, i32, vp]
    L.quantize_fp8_channel.restype = i32
    L.quantize_fp8_channel.argtypes = [vp, i64, i64, i32, vp, vp, i32, vp]
    L.gemm_fp8_splitk.restype = i32
    L.gemm_fp8_splitk.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp, i64, vp]
    L.gemm_fp8_splitk_noalloc.restype = i32
    L.gemm_fp8_splitk_noalloc.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.gemm_fp8_splitk_noalloc_max_bytes.restype = i64
    L.gemm_fp8_splitk_noalloc_max_bytes.argtypes = []
    L.gemm_f16_splitk.restype = i32
    L.gemm_f16_splitk.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, i64, vp]
    L.gemm_splitk_plan.restype = i32
    L.gemm_splitk_plan.argtypes = [i32, i32, i64, i64, i64, i32, i32, ctypes.c_char_p, i32,
                                   ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.gemm_f16_guarded.restype = i32
    L.gemm_f16_guarded.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, vp, i64, vp]
    L.gemm_f16_guarded_workspace_size.restype = i64
    L.gemm_f16_guarded_workspace_size.argtypes = [i64, i64, i64]
    L.gemm_select_config_fmt.restype = i32
    L.gemm_select_config_fmt.argtypes = [i32, i32, i64, i64, i64, i32, i32, ctypes.c_char_p, i32]
    L.gemm_f16_bt.restype = i32
    L.gemm_f16_bt.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp]
    L.gemm_fp8_scaled_bt.restype = i32
    L.gemm_fp8_scaled_bt.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.quantize_fp8_transposed.restype = i32
    L.quantize_fp8_transposed.argtypes = [vp, i64, i64, vp, vp, vp]
    L.gemm_select_config_bt.restype = i32
    L.gemm_select_config_bt.argtypes = [i32, i32, i64, i64, i64, ctypes.c_char_p, i32]
    L.gemm_fp8_fmt_bt.restype = i32
    L.gemm_fp8_fmt_bt.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.quantize_fp8_transposed_fmt.restype = i32
    L.quantize_fp8_transposed_fmt.argtypes = [vp, i64, i64, vp, vp, i32, vp]
    L.pack_b_kmajor.restype = i32
    L.pack_b_kmajor.argtypes = [vp, i64, i64, i32, vp, vp]
    L.gemm_fp8_splitk_bt.restype = i32
    L.gemm_fp8_splitk_bt.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, i64, vp]
    L.gemm_f16_splitk_bt.restype = i32
    L.gemm_f16_splitk_bt.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, i64, vp]
    L.gemm_splitk_plan_bt.restype = i32
    L.gemm_splitk_plan_bt.argtypes = [i32, i32, i64, i64, i64, ctypes.c_char_p, i32, ctypes.POINTER(i32),
                                      ctypes.POINTER(i64)]
    L.amax_quantize_fp8_pair.restype = i32
    L.amax_quantize_fp8_pair.argtypes = [vp, i64, vp, i64, i32, i32, vp, vp, vp, vp, vp, i64, vp]
    L.amax_quantize_fp8_pair_bt.restype = i32
    L.amax_quantize_fp8_pair_bt.argtypes = [vp, i64, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, i64, vp]
    L.amax_quantize_fp8_pair_workspace_size.restype = i64
    L.amax_quantize_fp8_pair_workspace_size.argtypes = []
    L.gemm_fp8_exact.restype = i32
    L.gemm_fp8_exact.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.gemm_fp8_exact_bt.restype = i32
    L.gemm_fp8_exact_bt.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.gemm_select_config_exact.restype = i32
    L.gemm_select_config_exact.argtypes = [i32, i64, i64, i64, i32, i32, i32, ctypes.c_char_p, i32]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().gemm_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != GEMM_OK:
        raise GemmError(status, what)


def _torch():
    import torch
    return torch


def _stream_handle(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libgemm takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libgemm takes contiguous (row-major) tensors")
    return t.data_ptr()


def _out_dtype(C, out_fmt=None):
    torch = _torch()
    if C.dtype == torch.float32:
        return OUT_F32
    if C.dtype == torch.float16:
        return OUT_F16
    if C.dtype == torch.float8_e5m2 or (C.dtype == torch.uint8 and out_fmt == FMT_E5M2):
        return OUT_E5M2
    if C.dtype in (torch.uint8, torch.float8_e4m3fn):
        return OUT_E4M3
    raise ValueError(f"unsupported output dtype {C.dtype}")


def _dims(A, B, C):
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B and C must be 2-D")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    return M, N, K


def _dims_bt(A, Bt, C):
    if A.dim() != 2 or Bt.dim() != 2 or C.dim() != 2:
        raise ValueError("A, Bt and C must be 2-D")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A{tuple(A.shape)} Bt{tuple(Bt.shape)} C{tuple(C.shape)}")
    return M, N, K


def gemm_f16_bt(A, Bt, C, stream=None):
    """C = A @ Bt.T for float16 A[M,K] and a K-major weight Bt[N,K]; C float32 or float16 [M,N]."""
    torch = _torch()
    if A.dtype != torch.float16 or Bt.dtype != torch.float16:
        raise ValueError("gemm_f16_bt takes float16 operands")
    M, N, K = _dims_bt(A, Bt, C)
    _check(lib().gemm_f16_bt(_ptr(A), _ptr(Bt), _ptr(C), _out_dtype(C), M, N, K, _stream_handle(stream)),
           "gemm_f16_bt")
    return C


def gemm_f16(A, B, C, stream=None):
    """C = A @ B for float16 A[M,K], B[K,N]; C float32 or float16 [M,N]."""
    torch = _torch()
    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise ValueError("gemm_f16 takes float16 operands")
    M, N, K = _dims(A, B, C)
    _check(lib().gemm_f16(_ptr(A), _ptr(B), _ptr(C), _out_dtype(C), M, N, K, _stream_handle(stream)), "gemm_f16")
    return C


def _u8(t, fmt=None):
    """The uint8 view of FP8 codes. A torch float8 tensor must be of format
    fmt when one is given (FMT_E4M3 / FMT_E5M2): its bits are not re-encoded."""
    torch = _torch()
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        have = FMT_E5M2 if t.dtype == torch.float8_e5m2 else FMT_E4M3
        if fmt is not None and int(fmt) != have:
            want = "E5M2" if int(fmt) == FMT_E5M2 else "E4M3"
            raise ValueError(f"a {t.dtype} tensor was passed where {want} codes are expected")
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError("FP8 tensors must be uint8 codes or torch float8 tensors")
    return t


def gemm_fp8_scaled(A, B, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """C = (sA*A) @ (sB*B) for E4M3 A[M,K], B[K,N]; sA, sB (and sOut for an
    FP8 C) are one-element float32 device tensors."""
    A, B = _u8(A, FMT_E4M3), _u8(B, FMT_E4M3)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    _check(lib().gemm_fp8_scaled(_ptr(A), _ptr(B), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv), out, M, N, K,
                                 _stream_handle(stream)), "gemm_fp8_scaled")
    return C


def gemm_fp8_scaled_bt(A, Bt, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_scaled with B given K-major: C = (sA*A) @ (sB*Bt).T for E4M3
    A[M,K] and Bt[N,K]."""
    A, Bt = _u8(A, FMT_E4M3), _u8(Bt, FMT_E4M3)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims_bt(A, Bt, Cv)
    _check(lib().gemm_fp8_scaled_bt(_ptr(A), _ptr(Bt), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv), out, M, N, K,
                                    _stream_handle(stream)), "gemm_fp8_scaled_bt")
    return C


def gemm_fp8_fmt_bt(A, fmt_a, Bt, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_scaled_bt with A in FP8 format fmt_a and Bt in fmt_b (FMT_E4M3 / FMT_E5M2)."""
    A, Bt = _u8(A, fmt_a), _u8(Bt, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims_bt(A, Bt, Cv)
    _check(lib().gemm_fp8_fmt_bt(_ptr(A), int(fmt_a), _ptr(Bt), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv),
                                 out, M, N, K, _stream_handle(stream)), "gemm_fp8_fmt_bt")
    return C


def quantize_fp8_transposed_fmt(x, scale, fmt, q=None, stream=None):
    """quantize_fp8_transposed into FP8 format fmt (FMT_E4M3 / FMT_E5M2)."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("quantize_fp8_transposed_fmt takes float32 input")
    rows, cols = _rows_cols(x)
    if q is None:
        q = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    qv = _u8(q, fmt)
    if qv.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib().quantize_fp8_transposed_fmt(_ptr(x), rows, cols, _ptr(scale), _ptr(qv), int(fmt),
                                             _stream_handle(stream)), "quantize_fp8_transposed_fmt")
    return q


def pack_b_kmajor(B, Bt=None, stream=None):
    """The K-major copy Bt[N, K] of a row-major weight B[K, N] (float16, or
    FP8 codes as uint8 / torch float8), made once on the GPU."""
    torch = _torch()
    if B.dim() != 2:
        raise ValueError("pack_b_kmajor takes a 2-D B")
    es = B.element_size()
    if es not in (1, 2):
        raise ValueError("pack_b_kmajor takes 1- or 2-byte elements")
    K, N = int(B.shape[0]), int(B.shape[1])
    if Bt is None:
        Bt = torch.empty((N, K), dtype=B.dtype, device=B.device)
    if tuple(Bt.shape) != (N, K) or Bt.element_size() != es:
        raise ValueError("Bt must be [N, K] with B's element size")
    _check(lib().pack_b_kmajor(_ptr(B), K, N, es, _ptr(Bt), _stream_handle(stream)), "pack_b_kmajor")
    return Bt


def quantize_fp8_transposed(x, scale, q=None, stream=None):
    """E4M3 codes of x / scale for a 2-D float32 x[rows, cols], written
    transposed: q[cols, rows] (uint8)."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("quantize_fp8_transposed takes float32 input")
    rows, cols = _rows_cols(x)
    if q is None:
        q = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    qv = _u8(q, FMT_E4M3)
    if qv.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib().quantize_fp8_transposed(_ptr(x), rows, cols, _ptr(scale), _ptr(qv), _stream_handle(stream)),
           "quantize_fp8_transposed")
    return q


def gemm_fp8_fmt(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_scaled with A in FP8 format fmt_a and B in fmt_b (FMT_E4M3 / FMT_E5M2)."""
    A, B = _u8(A, fmt_a), _u8(B, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    _check(lib().gemm_fp8_fmt(_ptr(A), int(fmt_a), _ptr(B), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv),
                              out, M, N, K, _stream_handle(stream)), "gemm_fp8_fmt")
    return C


def gemm_fp8_channel(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_fmt with per-channel scales: sA float32[M] (one per row of A),
    sB float32[N] (one per column of B); sOut stays one element."""
    A, B = _u8(A, fmt_a), _u8(B, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    torch = _torch()
    for name, s, n in (("sA", sA, M), ("sB", sB, N)):
        if s.dtype != torch.float32 or s.numel() != n:
            raise ValueError(f"{name} must be float32 with one scale per channel ({n})")
    _check(lib().gemm_fp8_channel(_ptr(A), int(fmt_a), _ptr(B), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut),
                                  _ptr(Cv), out, M, N, K, _stream_handle(stream)), "gemm_fp8_channel")
    return C


def _rows_cols(x):
    if x.dim() != 2:
        raise ValueError("per-channel calls take a 2-D x")
    return int(x.shape[0]), int(x.shape[1])


def quantize_fp8_channel(x, scale, axis, fmt, q=None, stream=None):
    """FP8 codes of x[i,j] / scale[i] (axis AXIS_ROW) or / scale[j] (AXIS_COL)."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("quantize_fp8_channel takes float32 input")
    rows, cols = _rows_cols(x)
    if scale.dtype != torch.float32 or scale.numel() != (rows if axis == AXIS_ROW else cols):
        raise ValueError("one float32 scale per channel")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    qv = _u8(q, fmt)
    if qv.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib().quantize_fp8_channel(_ptr(x), rows, cols, int(axis), _ptr(scale), _ptr(qv), int(fmt),
                                      _stream_handle(stream)), "quantize_fp8_channel")
    return q


def amax_scale_channel_f32(x, axis, fmt, pow2, amax=None, scale=None, stream=None):
    """(amax, scale) per row (axis AXIS_ROW) or per column (AXIS_COL) of x."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("amax_scale_channel_f32 takes float32 input")
    rows, cols = _rows_cols(x)
    n = rows if axis == AXIS_ROW else cols
    if amax is None:
        amax = torch.empty(n, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(n, dtype=torch.float32, device=x.device)
    if amax.numel() != n or scale.numel() != n:
        raise ValueError("amax and scale need one element per channel")
    _check(lib().amax_scale_channel_f32(_ptr(x), rows, cols, int(axis), _ptr(amax), _ptr(scale), int(fmt),
                                        1 if pow2 else 0, _stream_handle(stream)), "amax_scale_channel_f32")
    return amax, scale


def splitk_plan(kind: int, out_dtype: int, M: int, N: int, K: int, fmt_a: int = 0, fmt_b: int = 0):
    """(configuration name, number of K ranges, workspace bytes) of the
    split-K entry points for this request (host-only query)."""
    buf = ctypes.create_string_buffer(64)
    sp = ctypes.c_int(0)
    wb = ctypes.c_int64(0)
    _check(lib().gemm_splitk_plan(kind, out_dtype, M, N, K, fmt_a, fmt_b, buf, 64, ctypes.byref(sp),
                                  ctypes.byref(wb)), "gemm_splitk_plan")
    return buf.value.decode(), sp.value, wb.value


def _workspace(kind, out, M, N, K, fa, fb, workspace, device):
    if workspace is not None:
        return workspace
    _, _, nbytes = splitk_plan(kind, out, M, N, K, fa, fb)
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def gemm_fp8_splitk(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, workspace=None, stream=None, out_fmt=None):
    """gemm_fp8_fmt that splits K over a workspace when the shape has too few
    output tiles; workspace=None allocates one of the planned size."""
    A, B = _u8(A, fmt_a), _u8(B, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    ws, nbytes = _ws_args(_workspace(KIND_FP8, out, M, N, K, int(fmt_a), int(fmt_b), workspace, C.device))
    _check(lib().gemm_fp8_splitk(_ptr(A), int(fmt_a), _ptr(B), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv),
                                 out, M, N, K, ws, nbytes, _stream_handle(stream)), "gemm_fp8_splitk")
    return C


def gemm_fp8_splitk_noalloc(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_splitk with the partial sums in the library's own per-GPU
    array (no workspace, nothing allocated); calls that overlap on one GPU
    race."""
    A, B = _u8(A, fmt_a), _u8(B, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    _check(lib().gemm_fp8_splitk_noalloc(_ptr(A), int(fmt_a), _ptr(B), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut),
                                         _ptr(Cv), out, M, N, K, _stream_handle(stream)), "gemm_fp8_splitk_noalloc")
    return C


def gemm_fp8_splitk_noalloc_max_bytes() -> int:
    return int(lib().gemm_fp8_splitk_noalloc_max_bytes())


def gemm_f16_splitk(A, B, C, workspace=None, stream=None):
    """gemm_f16 that splits K over a workspace when the shape has too few
    output tiles; workspace=None allocates one of the planned size."""
    out = _out_dtype(C)
    if out not in (OUT_F32, OUT_F16):
        raise ValueError("gemm_f16 writes float32 or float16")
    M, N, K = _dims(A, B, C)
    ws, nbytes = _ws_args(_workspace(KIND_F16, out, M, N, K, 0, 0, workspace, C.device))
    _check(lib().gemm_f16_splitk(_ptr(A), _ptr(B), _ptr(C), out, M, N, K, ws, nbytes, _stream_handle(stream)),
           "gemm_f16_splitk")
    return C


def guarded_workspace_size(M: int, N: int, K: int) -> int:
    n = int(lib().gemm_f16_guarded_workspace_size(M, N, K))
    _check(n if n < 0 else 0, "gemm_f16_guarded_workspace_size")
    return n


def gemm_f16_guarded(A, B, C, scale=None, workspace=None, stream=None):
    """C = A @ B for float32 A[M,K], B[K,N] through the FP16 GEMM under the
    dynamic-range guard; returns (C, scale) with scale the one-element s."""
    torch = _torch()
    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise ValueError("gemm_f16_guarded takes float32 A and B")
    out = _out_dtype(C)
    if out not in (OUT_F32, OUT_F16):
        raise ValueError("gemm_f16_guarded writes float32 or float16")
    M, N, K = _dims(A, B, C)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=C.device)
    if workspace is None:
        workspace = torch.empty(guarded_workspace_size(M, N, K), dtype=torch.uint8, device=C.device)
    _check(lib().gemm_f16_guarded(_ptr(A), _ptr(B), _ptr(C), out, M, N, K, _ptr(scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "gemm_f16_guarded")
    return C, scale


def quantize_fp8(x, scale, q=None, stream=None):
    """E4M3 codes of x / scale (uint8, same shape as x)."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("quantize_fp8 takes float32 input")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    qv = _u8(q, FMT_E4M3)
    if qv.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib().quantize_fp8(_ptr(x), x.numel(), _ptr(scale), _ptr(qv), _stream_handle(stream)), "quantize_fp8")
    return q


def quantize_fp8_fmt(x, scale, fmt, q=None, stream=None):
    """FP8 codes (format fmt) of x / scale (uint8, same shape as x)."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("quantize_fp8_fmt takes float32 input")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    qv = _u8(q, fmt)
    if qv.numel() != x.numel():
        raise ValueError("q must have as many elements as x")
    _check(lib().quantize_fp8_fmt(_ptr(x), x.numel(), _ptr(scale), _ptr(qv), int(fmt), _stream_handle(stream)),
           "quantize_fp8_fmt")
    return q


def amax_scale_f32(x, fmt, pow2, amax=None, scale=None, stream=None):
    """(amax, scale) with the scale for FP8 format fmt: amax / fmax, or with pow2
    the smallest power of two s with amax / s <= fmax."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("amax_scale_f32 takes float32 input")
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().amax_scale_f32(_ptr(x), x.numel(), _ptr(amax), _ptr(scale), int(fmt), 1 if pow2 else 0,
                                _stream_handle(stream)), "amax_scale_f32")
    return amax, scale


def amax_f32(x, amax=None, scale=None, stream=None):
    """(amax, scale): max|x| and max|x|/448 (1 if that is 0) as 1-element device tensors."""
    torch = _torch()
    if x.dtype != torch.float32:
        raise ValueError("amax_f32 takes float32 input")
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(lib().amax_f32(_ptr(x), x.numel(), _ptr(amax), _ptr(scale), _stream_handle(stream)), "amax_f32")
    return amax, scale


def select_config(kind: int, out_dtype: int, M: int, N: int, K: int) -> str:
    buf = ctypes.create_string_buffer(128)
    _check(lib().gemm_select_config(kind, out_dtype, M, N, K, buf, len(buf)), "gemm_select_config")
    return buf.value.decode()


def select_config_fmt(kind: int, out_dtype: int, M: int, N: int, K: int, fmt_a: int, fmt_b: int) -> str:
    buf = ctypes.create_string_buffer(128)
    _check(lib().gemm_select_config_fmt(kind, out_dtype, M, N, K, int(fmt_a), int(fmt_b), buf, len(buf)),
           "gemm_select_config_fmt")
    return buf.value.decode()


def select_config_bt(kind: int, out_dtype: int, M: int, N: int, K: int) -> str:
    """The configuration gemm_f16_bt (kind 0) or gemm_fp8_scaled_bt (kind 1) would launch."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().gemm_select_config_bt(kind, out_dtype, M, N, K, buf, len(buf)), "gemm_select_config_bt")
    return buf.value.decode()


def splitk_plan_bt(kind: int, out_dtype: int, M: int, N: int, K: int):
    """splitk_plan for the K-major split-K calls."""
    buf = ctypes.create_string_buffer(64)
    sp = ctypes.c_int(0)
    wb = ctypes.c_int64(0)
    _check(lib().gemm_splitk_plan_bt(kind, out_dtype, M, N, K, buf, 64, ctypes.byref(sp), ctypes.byref(wb)),
           "gemm_splitk_plan_bt")
    return buf.value.decode(), sp.value, wb.value


def _workspace_bt(kind, out, M, N, K, workspace, device):
    if workspace is not None:
        return workspace
    _, _, nbytes = splitk_plan_bt(kind, out, M, N, K)
    if nbytes == 0:
        return None
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def gemm_fp8_splitk_bt(A, Bt, sA, sB, C, sOut=None, workspace=None, stream=None, out_fmt=None):
    """gemm_fp8_scaled_bt that splits K over a workspace for mid-M shapes;
    workspace=None allocates one of the planned size."""
    A, Bt = _u8(A, FMT_E4M3), _u8(Bt, FMT_E4M3)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims_bt(A, Bt, Cv)
    ws, nbytes = _ws_args(_workspace_bt(KIND_FP8, out, M, N, K, workspace, C.device))
    _check(lib().gemm_fp8_splitk_bt(_ptr(A), _ptr(Bt), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv), out, M, N, K, ws,
                                    nbytes, _stream_handle(stream)), "gemm_fp8_splitk_bt")
    return C


def gemm_f16_splitk_bt(A, Bt, C, workspace=None, stream=None):
    """gemm_f16_bt that splits K over a workspace for mid-M shapes."""
    torch = _torch()
    if A.dtype != torch.float16 or Bt.dtype != torch.float16:
        raise ValueError("gemm_f16_splitk_bt takes float16 operands")
    M, N, K = _dims_bt(A, Bt, C)
    out = _out_dtype(C)
    ws, nbytes = _ws_args(_workspace_bt(KIND_F16, out, M, N, K, workspace, C.device))
    _check(lib().gemm_f16_splitk_bt(_ptr(A), _ptr(Bt), _ptr(C), out, M, N, K, ws, nbytes, _stream_handle(stream)),
           "gemm_f16_splitk_bt")
    return C


def gemm_fp8_exact(A, fmt_a, B, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_fmt with exact products and FP32 additions throughout (the
    codes widened to FP16 on the FP16 matrix cores, or the FP32-FMA decode
    kernels)."""
    A, B = _u8(A, fmt_a), _u8(B, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims(A, B, Cv)
    _check(lib().gemm_fp8_exact(_ptr(A), int(fmt_a), _ptr(B), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut), _ptr(Cv),
                                out, M, N, K, _stream_handle(stream)), "gemm_fp8_exact")
    return C


def gemm_fp8_exact_bt(A, fmt_a, Bt, fmt_b, sA, sB, C, sOut=None, stream=None, out_fmt=None):
    """gemm_fp8_exact with B given K-major as Bt[N,K]."""
    A, Bt = _u8(A, fmt_a), _u8(Bt, fmt_b)
    out = _out_dtype(C, out_fmt)
    Cv = _u8(C) if out in (OUT_E4M3, OUT_E5M2) else C
    M, N, K = _dims_bt(A, Bt, Cv)
    _check(lib().gemm_fp8_exact_bt(_ptr(A), int(fmt_a), _ptr(Bt), int(fmt_b), _ptr(sA), _ptr(sB), _ptr(sOut),
                                   _ptr(Cv), out, M, N, K, _stream_handle(stream)), "gemm_fp8_exact_bt")
    return C


def select_config_exact(out_dtype: int, M: int, N: int, K: int, fmt_a: int = 0, fmt_b: int = 0,
                        b_kmajor: int = 0) -> str:
    """The configuration gemm_fp8_exact (or, with b_kmajor, gemm_fp8_exact_bt) would launch."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().gemm_select_config_exact(out_dtype, M, N, K, int(fmt_a), int(fmt_b), int(b_kmajor), buf, len(buf)),
           "gemm_select_config_exact")
    return buf.value.decode()


def amax_quantize_fp8_pair(xa, xb, fmt=FMT_E4M3, pow2=False, amax=None, scale=None, qa=None, qb=None,
                           workspace=None, stream=None):
    """amax, scale and FP8 codes of two float32 tensors in two launches:
    returns (amax[2], scale[2], qa, qb), bit-identical to amax_scale_f32 and
    quantize_fp8_fmt on each. xb may be None (then amax and scale have one
    element and qb is None)."""
    torch = _torch()
    for name, x in (("xa", xa), ("xb", xb)):
        if x is not None and x.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    dev = xa.device
    two = xb is not None
    if amax is None:
        amax = torch.empty(2 if two else 1, dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty(2 if two else 1, dtype=torch.float32, device=dev)
    if qa is None:
        qa = torch.empty(xa.shape, dtype=torch.uint8, device=dev)
    if two and qb is None:
        qb = torch.empty(xb.shape, dtype=torch.uint8, device=dev)
    qav = _u8(qa, fmt)
    qbv = _u8(qb, fmt) if two else None
    if qav.numel() != xa.numel() or (two and qbv.numel() != xb.numel()):
        raise ValueError("q must have as many elements as its x")
    if amax.numel() < (2 if two else 1) or scale.numel() < (2 if two else 1):
        raise ValueError("amax and scale need one element per tensor")
    if workspace is None:
        workspace = torch.empty(int(lib().amax_quantize_fp8_pair_workspace_size()), dtype=torch.uint8, device=dev)
    _check(lib().amax_quantize_fp8_pair(_ptr(xa), xa.numel(), _ptr(xb) if two else None, xb.numel() if two else 0,
                                        int(fmt), 1 if pow2 else 0, _ptr(amax), _ptr(scale), _ptr(qav),
                                        _ptr(qbv) if two else None, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "amax_quantize_fp8_pair")
    return amax, scale, qa, qb


def amax_quantize_fp8_pair_bt(xa, xb, fmt=FMT_E4M3, pow2=False, amax=None, scale=None, qa=None, qbt=None,
                              workspace=None, stream=None):
    """amax_quantize_fp8_pair for a row-major float32 xb[K, N] whose codes are
    written K-major: returns (amax[2], scale[2], qa, qbt) with qbt[N, K] the
    transpose of amax_quantize_fp8_pair's qb, for the gemm_*_bt calls."""
    torch = _torch()
    for name, x in (("xa", xa), ("xb", xb)):
        if x.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if xb.dim() != 2 or not xb.is_contiguous():
        raise ValueError("xb must be a contiguous [K, N] matrix")
    K, N = xb.shape
    dev = xa.device
    if amax is None:
        amax = torch.empty(2, dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty(2, dtype=torch.float32, device=dev)
    if qa is None:
        qa = torch.empty(xa.shape, dtype=torch.uint8, device=dev)
    if qbt is None:
        qbt = torch.empty((N, K), dtype=torch.uint8, device=dev)
    qav, qbv = _u8(qa, fmt), _u8(qbt, fmt)
    if qav.numel() != xa.numel() or qbv.numel() != xb.numel():
        raise ValueError("q must have as many elements as its x")
    if amax.numel() < 2 or scale.numel() < 2:
        raise ValueError("amax and scale need one element per tensor")
    if workspace is None:
        workspace = torch.empty(int(lib().amax_quantize_fp8_pair_workspace_size()), dtype=torch.uint8, device=dev)
    _check(lib().amax_quantize_fp8_pair_bt(_ptr(xa), xa.numel(), _ptr(xb), K, N, int(fmt), 1 if pow2 else 0,
                                           _ptr(amax), _ptr(scale), _ptr(qav), _ptr(qbv), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream_handle(stream)),
           "amax_quantize_fp8_pair_bt")
    return amax, scale, qa, qbt
