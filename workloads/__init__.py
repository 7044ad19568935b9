"""Seeded synthetic inputs for the GEMM workloads.

Shared by the tests, the benchmark and the smoke check; imported by neither
the oracle nor the product library. It holds no step of the method (no amax,
no scaling, no quantization, no products): only random numbers and their
rounding to the storage type the workload names.

Every generator is seeded with ``numpy.random.default_rng([cfg, tensor, variant])``
(cfg: workload number below; tensor: A=0, B=1; variant: the swept size, else 0)
so that the oracle and the GPU see the same bits.

Workloads (shapes and distributions of the FP8/FP16 GEMM pages' examples):
  1  FP16 256^3, A,B ~ U(-1,1) rounded to fp16, FP32 output
  2  FP8 1024^3 from FP32 A,B ~ N(0,1), per-tensor scales, FP32 output
  3  FP16 decode M in {1,4,16}, K=4096, N=12288: A ~ N(0,1), B ~ N(0, 0.02^2), fp16 output
  4  FP8 N=K=4096, M in {1,63,65,127,129,3000,4096}: N(0,1) with 0.1% outliers x50,
     FP8 output with its own output scale
  5  FP8 16384x12288x4096 and FP16 8192^3 from N(0,1), fp16 output
  0  FP16 4096^3 from N(0,1), fp16 output
"""
from dataclasses import dataclass

import numpy as np

OUT_F32 = 0
OUT_F16 = 1
OUT_E4M3 = 2


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int          # seed component
    variant: int      # seed component (swept size), 0 if none
    kind: str         # "f16" (fp16 operands) or "fp8" (FP32 operands to be quantized)
    M: int
    N: int
    K: int
    out: int          # OUT_F32 / OUT_F16 / OUT_E4M3
    dist: str         # "uniform", "normal", "normal_outliers", "decode"


def _w(name, cfg, variant, kind, M, N, K, out, dist):
    return Workload(name, cfg, variant, kind, M, N, K, out, dist)


C1 = _w("fp16_256^3_f32out", 1, 0, "f16", 256, 256, 256, OUT_F32, "uniform")
C2 = _w("fp8_1024^3_f32out", 2, 0, "fp8", 1024, 1024, 1024, OUT_F32, "normal")
C3 = [_w(f"fp16_decode_M{m}_K4096_N12288", 3, m, "f16", m, 12288, 4096, OUT_F16, "decode")
      for m in (1, 4, 16)]
C4 = [_w(f"fp8_M{m}_N4096_K4096_fp8out", 4, m, "fp8", m, 4096, 4096, OUT_E4M3, "normal_outliers")
      for m in (1, 63, 65, 127, 129, 3000, 4096)]
C5_FP8 = _w("fp8_16384x12288x4096_f16out", 5, 0, "fp8", 16384, 12288, 4096, OUT_F16, "normal")
C5_F16 = _w("fp16_8192^3_f16out", 5, 8192, "f16", 8192, 8192, 8192, OUT_F16, "normal")
M0 = _w("fp16_4096^3_f16out", 0, 0, "f16", 4096, 4096, 4096, OUT_F16, "normal")

ALL = [C1, C2, *C3, *C4, C5_FP8, C5_F16, M0]


def rng(cfg: int, tensor: int, variant: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg, tensor, variant])


def _outliers(x: np.ndarray, g: np.random.Generator, frac: float = 0.001, factor: float = 50.0):
    """Multiply round(frac * numel) distinct positions by factor (in place)."""
    flat = x.reshape(-1)
    k = int(round(frac * flat.size))
    if k:
        idx = g.choice(flat.size, k, replace=False)
        flat[idx] *= np.float32(factor)
    return x


def operand(w: Workload, tensor: int, shape=None) -> np.ndarray:
    """Operand A (tensor=0, [M,K]) or B (tensor=1, [K,N]) of workload w.

    fp16 workloads return float16 arrays (RNE from float32 draws); fp8
    workloads return the FP32 tensor that the method quantizes.
    """
    if shape is None:
        shape = (w.M, w.K) if tensor == 0 else (w.K, w.N)
    g = rng(w.cfg, tensor, w.variant)
    if w.dist == "uniform":
        x = g.uniform(-1.0, 1.0, shape).astype(np.float32)
    elif w.dist == "normal":
        x = g.standard_normal(shape, dtype=np.float32)
    elif w.dist == "decode":
        x = g.standard_normal(shape, dtype=np.float32)
        if tensor == 1:
            x *= np.float32(0.02)
    elif w.dist == "normal_outliers":
        x = _outliers(g.standard_normal(shape, dtype=np.float32), g)
    else:
        raise ValueError(w.dist)
    if w.kind == "f16":
        return x.astype(np.float16)
    return x


def random_e4m3_codes(shape, seed, finite=True) -> np.ndarray:
    """Uniformly random E4M3 codes over the whole table (NaN codes excluded
    when finite=True): zeros, subnormals, +-448 and both signs all occur."""
    g = np.random.default_rng([9000, seed])
    c = g.integers(0, 256, size=shape, dtype=np.uint16).astype(np.uint8)
    if finite:
        nan = (c & 0x7F) == 0x7F
        c[nan] = c[nan] ^ 0x01  # 0x7F -> 0x7E, 0xFF -> 0xFE
    return c


def random_e5m2_codes(shape, seed):
    """Uniformly random finite E5M2 codes (infinities and NaNs excluded)."""
    g = np.random.default_rng([9100, seed])
    c = g.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) > 0x7B, c & 0xBB, c).astype(np.uint8)


def random_f16(shape, seed, lo=-1.0, hi=1.0) -> np.ndarray:
    g = np.random.default_rng([9001, seed])
    return g.uniform(lo, hi, size=shape).astype(np.float16)


def random_normal_f32(shape, seed) -> np.ndarray:
    g = np.random.default_rng([9002, seed])
    return g.standard_normal(shape, dtype=np.float32)


def normal_with_outliers_f32(shape, seed) -> np.ndarray:
    """N(0,1) FP32 with 0.1% of the positions multiplied by 50 (the outlier
    mix of the M-sweep workload)."""
    g = np.random.default_rng([9003, seed])
    return _outliers(g.standard_normal(shape, dtype=np.float32), g)
