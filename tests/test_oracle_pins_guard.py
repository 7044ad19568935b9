"""Pins of the oracle's FP16 dynamic-range guard (CPU only): the scale
against closed forms, the scaled FP16 conversion against numpy's IEEE
float32 arithmetic and float16 cast, the product bound the guard exists for,
and the guarded product against the exact product of the FP32 inputs within
the FP16 rounding bound."""
import numpy as np
import pytest

import oracle as orc
import workloads as wl

F16_MAX = 65504.0


def test_guard_scale_closed_forms():
    assert orc.guard_scale(255.0, 256.0) == 1.0                  # 65280 <= 65504: no scaling
    assert orc.guard_scale(1.0, F16_MAX) == 1.0
    for k in range(9, 40):
        # 65504 * 2^-(2k) is exact in FP32 (65504 has 11 significant bits)
        assert orc.guard_scale(2.0 ** k, 2.0 ** k) == np.float32(F16_MAX * 2.0 ** (-2 * k))
    assert orc.guard_scale(3.0e4, 3.0) == np.float32(F16_MAX / 9.0e4)
    assert orc.guard_scale(0.0, 7.0) == 1.0                      # empty or zero operand
    assert np.isnan(np.float32(np.nan)) and orc.guard_scale(np.nan, 1.0) == 1.0
    assert orc.guard_scale(np.inf, 1.0) == 0.0
    assert orc.guard_scale(3.0e38, 3.0e38) == 0.0                # the quotient underflows FP32


def test_guard_to_f16_unscaled_is_numpy_cast():
    x = np.concatenate([wl.random_normal_f32((5000,), 1) * np.float32(3e4),
                        np.array([65504, 65519.99, 65520, -1e6, 6e-8, 2.9e-8, 0.0, -0.0], np.float32)])
    got = orc.guard_to_f16(x, 1.0)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("s", [0.25, 0.5, 0.3, 0.0123, 1e-6])
def test_guard_to_f16_matches_ieee_float32_steps(s):
    """r = sqrt(s) and x * r, each correctly rounded in float32 (numpy), then the float16 cast."""
    x = np.concatenate([wl.random_normal_f32((4000,), 2) * np.float32(1e5),
                        np.array([1e9, -7.5e4, 1e-30, 0.0], np.float32)])
    s32 = np.float32(s)
    r = np.sqrt(s32)
    with np.errstate(over="ignore"):
        ref = (x * r).astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.guard_to_f16(x, s32), ref)
    if s == 0.25:
        assert r == np.float32(0.5)


def test_guard_bounds_every_scaled_product():
    """max|a'| * max|b'| <= 65504 (up to the FP32/FP16 roundings of the scaled
    values): the property the guard is for."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        a_max = np.float32(np.exp2(rng.uniform(0, 30)))
        b_max = np.float32(np.exp2(rng.uniform(0, 30)))
        s = orc.guard_scale(a_max, b_max)
        a16 = orc.f16_decode(orc.guard_to_f16(np.array([a_max]), s))[0]
        b16 = orc.f16_decode(orc.guard_to_f16(np.array([b_max]), s))[0]
        if np.isfinite(a16) and np.isfinite(b16):
            assert a16 * b16 <= F16_MAX * (1 + 2.0 ** -9)
        # both operands stay finite whenever their ratio is within the FP16 range
        if max(a_max / b_max, b_max / a_max) <= F16_MAX / 2:
            assert np.isfinite(a16) and np.isfinite(b16)


def test_guarded_product_recovers_the_fp32_product():
    """A with outliers beyond the FP16 range (which a plain cast turns into
    inf), B ~ N(0,1): the guarded result (sqrt(s) A)_16 (sqrt(s) B)_16 / s is
    finite and within the FP16 rounding bound of the exact product. (The
    scale bounds products; it keeps both operands finite while
    max|A| / max|B| <= 65504, as here: 2e5 against about 4.)"""
    M, N, K = 24, 40, 256
    a = wl.random_normal_f32((M, K), 4)
    a[3, 7] = 2.0e5
    a[10, 100] = -1.5e5
    b = wl.random_normal_f32((K, N), 5)
    assert orc.amax(a) / orc.amax(b) <= F16_MAX
    with np.errstate(over="ignore"):
        assert np.isinf(a.astype(np.float16)).any()
    s = orc.guard_scale(orc.amax(a), orc.amax(b))
    assert s < 1
    a16, b16 = orc.guard_to_f16(a, s), orc.guard_to_f16(b, s)
    R, S = orc.gemm(orc.FMT_F16, a16, b16)
    V = R / float(s)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    bound = (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64)) * (2.0 ** -10 + 2.0 ** -20)
    assert np.all(np.isfinite(V))
    assert np.all(np.abs(V - exact) <= bound)
