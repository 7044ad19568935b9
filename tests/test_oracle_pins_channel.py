"""Pins of the oracle's per-channel scaling (CPU only): channel maxima against
numpy's reductions, scales against closed forms, per-channel quantization
against torch's float8 casts of the FP32 quotient, the row/column symmetry,
the half-step dequantization bound, and the scaled GEMM against a float64
matmul of the dequantized, scaled operands."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from parity import scale_grid, ulp_e4m3, ulp_e5m2

TORCH_FP8 = {orc.FMT_E4M3: torch.float8_e4m3fn, orc.FMT_E5M2: torch.float8_e5m2}
FMAX = {orc.FMT_E4M3: 448.0, orc.FMT_E5M2: 57344.0}


def torch_encode(x32, fmt):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()


def channel_data(rows, cols, seed):
    """Normal data whose rows span 2^-20 .. 2^20 in magnitude, so that using
    another channel's scale changes almost every code."""
    x = wl.random_normal_f32((rows, cols), seed)
    e = np.random.default_rng(seed + 1).integers(-20, 21, size=(rows, 1))
    return (x * np.exp2(e)).astype(np.float32)


# -------------------------------------------------------------------- amax

@pytest.mark.parametrize("axis", [0, 1])
def test_amax_channel_matches_numpy(axis):
    x = channel_data(37, 53, 3)
    x[5, 7] = np.inf
    x[11, 2] = -np.inf
    x[20, 30] = np.nan
    got = orc.amax_channel(x, axis)
    ref = np.max(np.abs(x), axis=1 - axis)          # numpy propagates NaN
    assert got.dtype == np.float32 and got.shape == ref.shape
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got[20 if axis == 0 else 30])


def test_amax_channel_empty_channels():
    assert np.array_equal(orc.amax_channel(np.zeros((4, 0), np.float32), 0), np.zeros(4, np.float32))
    assert np.array_equal(orc.amax_channel(np.zeros((0, 3), np.float32), 1), np.zeros(3, np.float32))
    assert orc.amax_channel(np.zeros((0, 3), np.float32), 0).shape == (0,)


# ------------------------------------------------------------------- scale

def test_scale_channel_closed_forms():
    k = np.arange(-30, 31)
    for fmt in (orc.FMT_E4M3, orc.FMT_E5M2):
        a = (FMAX[fmt] * np.exp2(k)).astype(np.float32)
        # amax = fmax * 2^k: the quotient and the power-of-two scale are 2^k
        assert np.array_equal(orc.scale_channel(a, fmt, False), np.exp2(k).astype(np.float32))
        assert np.array_equal(orc.scale_channel(a, fmt, True), np.exp2(k).astype(np.float32))
        # just above fmax * 2^k: the next power of two
        up = np.nextafter(a, np.float32(np.inf))
        assert np.array_equal(orc.scale_channel(up, fmt, True), np.exp2(k + 1).astype(np.float32))
    special = np.array([0.0, np.inf, np.nan, 1.4e-45, 3.0], np.float32)
    s = orc.scale_channel(special, orc.FMT_E4M3, True)
    assert s[0] == 1.0 and s[1] == np.inf and np.isnan(s[2])
    assert s[3] == np.float32(2.0 ** -149) and s[4] == np.float32(2.0 ** -7)   # 3 / 2^-7 = 384 <= 448 < 768
    s = orc.scale_channel(special, orc.FMT_E4M3, False)
    assert s[0] == 1.0 and s[1] == np.inf and np.isnan(s[2]) and s[3] == 1.0   # 1.4e-45 / 448 underflows
    assert s[4] == np.float32(np.float32(3.0) / np.float32(448.0))


# ---------------------------------------------------------------- quantize

@pytest.mark.parametrize("fmt", [orc.FMT_E4M3, orc.FMT_E5M2])
@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_rows_matches_torch_cast_of_quotient(fmt, pow2):
    x = channel_data(64, 96, 17)
    s = orc.scale_channel(orc.amax_channel(x, 0), fmt, pow2)
    q = orc.quantize_channel(x, s, 0, fmt)
    quot = x / s[:, None]                            # IEEE float32 division, correctly rounded
    # in range up to the scale's own rounding (a few FP32 ulps above fmax, which
    # still rounds to fmax): torch's casts do not saturate, but need no saturation here
    assert np.all(np.abs(quot) <= FMAX[fmt] * (1 + 2.0 ** -20))
    assert np.array_equal(q, torch_encode(quot, fmt))


@pytest.mark.parametrize("fmt", [orc.FMT_E4M3, orc.FMT_E5M2])
def test_quantize_cols_is_transposed_rows(fmt):
    x = channel_data(80, 48, 23).T.copy()            # columns span the magnitudes
    s = orc.scale_channel(orc.amax_channel(x, 1), fmt, False)
    q = orc.quantize_channel(x, s, 1, fmt)
    assert np.array_equal(q, orc.quantize_channel(x.T.copy(), s, 0, fmt).T)
    assert np.array_equal(q, torch_encode(x / s[None, :], fmt))


@pytest.mark.parametrize("fmt", [orc.FMT_E4M3, orc.FMT_E5M2])
def test_quantize_channel_dequantizes_within_half_step(fmt):
    """|s_c * dec(q) - x| <= s_c * (ulp(x / s_c) / 2 + |x / s_c| * 2^-24): round
    to nearest in the FP8 format after one correctly rounded FP32 division."""
    x = channel_data(50, 70, 29)
    s = orc.scale_channel(orc.amax_channel(x, 0), fmt, False)
    q = orc.quantize_channel(x, s, 0, fmt)
    t = x.astype(np.float64) / s[:, None]
    ulp = ulp_e5m2 if fmt == orc.FMT_E5M2 else ulp_e4m3
    err = np.abs(orc.fp8_decode(q, fmt) * s[:, None] - x)
    assert np.all(err <= s[:, None] * (ulp(t) / 2 + np.abs(t) * 2.0 ** -24))


def test_quantize_channel_equal_scales_is_per_tensor():
    x = channel_data(33, 40, 31)
    s0 = np.float32(0.75)
    for axis, n in ((0, 33), (1, 40)):
        for fmt in (orc.FMT_E4M3, orc.FMT_E5M2):
            q = orc.quantize_channel(x, np.full(n, s0, np.float32), axis, fmt)
            assert np.array_equal(q, orc.quantize(x, s0, fmt))


def test_quantize_channel_rejects_wrong_scale_count():
    with pytest.raises(ValueError):
        orc.quantize_channel(np.zeros((3, 4), np.float32), np.ones(4, np.float32), 0)


# -------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("fa,fb", [(orc.FMT_E4M3, orc.FMT_E4M3), (orc.FMT_E5M2, orc.FMT_E4M3)])
def test_channel_scaled_gemm_is_matmul_of_scaled_operands(fa, fb):
    """diag(sA) (A B) diag(sB) = (diag(sA) A)(B diag(sB)): with power-of-two
    scales every term of one output carries the same exact factor, so the
    double sums agree exactly with a float64 matmul of the scaled operands."""
    M, N, K = 23, 31, 64
    enc = {orc.FMT_E4M3: wl.random_e4m3_codes, orc.FMT_E5M2: wl.random_e5m2_codes}
    ca, cb = enc[fa]((M, K), 5), enc[fb]((K, N), 6)
    rng = np.random.default_rng(7)
    sA = np.exp2(rng.integers(-8, 9, M)).astype(np.float32)
    sB = np.exp2(rng.integers(-8, 9, N)).astype(np.float32)
    R, _ = orc.gemm(fa, ca, cb, fmt_b=fb)
    lhs = scale_grid(sA, sB) * R
    rhs = (orc.fp8_decode(ca, fa) * sA[:, None].astype(np.float64)) @ \
          (orc.fp8_decode(cb, fb) * sB[None, :].astype(np.float64))
    assert np.array_equal(lhs, rhs)
