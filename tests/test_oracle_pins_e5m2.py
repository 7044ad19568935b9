"""Pins of the oracle's E5M2 codec, power-of-two scales and mixed-format GEMM
(CPU only), against the pages' printed values, torch's float8_e5m2 casts,
closed forms and exact rational sums."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_e5m2_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e5m2).to(torch.float64).numpy()


def torch_e5m2_encode_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


# ------------------------------------------------------------------ decode

def test_e5m2_pages_constants():
    g = json.load(open(GOLDEN))
    assert g["e5m2_bits"]["exponent"] == 5 and g["e5m2_bits"]["mantissa"] == 2
    dec = orc.e5m2_decode(ALL_CODES)
    finite = dec[np.isfinite(dec)]
    assert finite.max() == g["e5m2_max"]["value"] == 57344.0
    # 2 mantissa bits: 4 codes per binade above the subnormals
    assert dec[0x04] == 2.0 ** -14 and dec[0x08] == 2.0 ** -13 and dec[0x3C] == 1.0


def test_e5m2_decode_all_256_codes_vs_torch():
    ours = orc.e5m2_decode(ALL_CODES)
    ref = torch_e5m2_decode(ALL_CODES)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # inf and signed zero too


def test_e5m2_decode_structure():
    dec = orc.e5m2_decode(ALL_CODES)
    assert np.all(np.diff(dec[:0x7D]) > 0)          # 0x00..0x7B finite, 0x7C = +inf
    assert dec[0x01] == 2.0 ** -16 and dec[0x03] == 3 * 2.0 ** -16
    assert dec[0x7C] == np.inf and dec[0xFC] == -np.inf
    assert np.array_equal(dec[0x80:0xFD], -dec[0x00:0x7D])


# ------------------------------------------------------------------ encode

def test_e5m2_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) <= 0x7B], np.uint8)
    assert np.array_equal(orc.e5m2_encode(orc.e5m2_decode(codes)), codes)


def test_e5m2_encode_midpoints_ties_to_even():
    dec = orc.e5m2_decode(ALL_CODES)
    for c in range(0x7B):
        lo, hi = dec[c], dec[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        got = orc.e5m2_encode(np.array([mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]))
        assert got[0] == even and got[1] == (0x80 | even)
        assert got[2] == c and got[3] == c + 1


def test_e5m2_encode_special_values():
    v = np.array([-0.0, 0.0, 2.0 ** -17, 1.5 * 2.0 ** -17, 57344.0, 61439.0, 61440.0, 1e30, np.inf, -np.inf,
                  np.nan, 3.0, 3.5, 1.25])
    expect = [0x80, 0x00, 0x00, 0x01, 0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0x7F, 0x42, 0x43, 0x3D]
    assert list(orc.e5m2_encode(v)) == expect


def test_e5m2_encode_all_fp32_bit_patterns_vs_torch():
    """All 2^32 FP32 inputs. Below 61440 (57344 plus half its ulp) torch's RNE
    cast is the reference; from there on torch rounds to inf while the pages
    clamp to +-57344 (saturation); NaN gives the canonical 0x7F."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(chunk, dtype=np.uint32) + np.uint32(start)
        ours = orc.e5m2_encode_f32bits(bits)
        f = bits.view(np.float32)
        with np.errstate(invalid="ignore"):
            absf = np.abs(f)
        nan = np.isnan(f)
        inrange = (~nan) & (absf < 61440.0)
        ref = torch_e5m2_encode_f32(f)
        assert np.array_equal(ours[inrange], ref[inrange]), hex(start)
        big = (~nan) & (absf >= 61440.0)
        sat = np.where(np.signbit(f[big]), 0xFB, 0x7B).astype(np.uint8)
        assert np.array_equal(ours[big], sat), hex(start)
        assert np.all(ours[nan] == 0x7F), hex(start)


# ------------------------------------------------------------------ scales

def _pow2_scale_exact(a, fmax):
    """Smallest power of two 2^e (e >= -149) with a / 2^e <= fmax, by exact rationals."""
    r = Fraction(float(a)) / Fraction(fmax)
    e = r.numerator.bit_length() - r.denominator.bit_length() - 2
    while Fraction(2) ** e < r:
        e += 1
    while e > -149 and Fraction(2) ** (e - 1) >= r:
        e -= 1
    return max(e, -149)


def test_pow2_scale_definition_and_tightness():
    g = np.random.default_rng(11)
    a = np.concatenate([(g.random(3000) * 10.0 ** g.uniform(-44, 38, 3000)),
                        [448.0, 449.0, 896.0, 897.0, 57344.0, 57345.0, 1.0, 3.4e38, 1.4e-45, 1e-40]])
    a = a.astype(np.float32)
    a = a[(a > 0) & np.isfinite(a)]
    for fmt, fmax in ((orc.FMT_E4M3, 448.0), (orc.FMT_E5M2, 57344.0)):
        for x in a:
            s = float(orc.scale(x, fmt, pow2=True))
            m, _ = math.frexp(s)
            assert m == 0.5, (x, s)                                   # a power of two
            assert s == 2.0 ** _pow2_scale_exact(x, fmax), (x, s)
            assert Fraction(float(x)) / Fraction(s) <= fmax            # no saturation of the maximum
            if s > 2.0 ** -149:
                assert Fraction(float(x)) / Fraction(s / 2) > fmax     # and the smallest such


def test_scale_special_values_and_plain_e5m2():
    for fmt in (orc.FMT_E4M3, orc.FMT_E5M2):
        assert orc.scale(0.0, fmt, pow2=True) == 1.0
        assert orc.scale(np.inf, fmt, pow2=True) == np.inf
        assert np.isnan(orc.scale(np.nan, fmt, pow2=True))
    assert orc.scale(448.0, orc.FMT_E4M3, pow2=True) == 1.0
    assert orc.scale(448.0 * 1.0000001, orc.FMT_E4M3, pow2=True) == 2.0
    # plain E5M2 scale is the IEEE FP32 quotient amax / 57344, as for E4M3 with 448
    g = np.random.default_rng(12)
    a = (g.random(5000) * 10.0 ** g.uniform(-30, 30, 5000)).astype(np.float32)
    ref = (a / np.float32(57344.0)).astype(np.float32)
    ours = np.array([orc.scale(x, orc.FMT_E5M2) for x in a], np.float32)
    assert np.array_equal(ours.view(np.uint32), np.where(ref == 0, np.float32(1), ref).view(np.uint32))
    assert orc.scale(448.0, orc.FMT_E4M3) == orc.scale_from_amax(448.0)


# ---------------------------------------------------------------- quantize

def test_quantize_e5m2_vs_torch_division_and_cast():
    x = wl.random_normal_f32((400, 401), 21)
    x.reshape(-1)[::89] *= 1000.0
    s = orc.scale(orc.amax(x), orc.FMT_E5M2)
    q = orc.quantize(x, s, orc.FMT_E5M2)
    ref = (torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert q.reshape(-1)[np.argmax(np.abs(x))] & 0x7F == 0x7B      # the maximum lands on 57344


def test_quantize_pow2_scale_is_exact_exponent_shift():
    """With a power-of-two scale the FP32 quotient is exact (no rounding before
    the encode), so quantize equals encoding x * 2^-e in double directly."""
    x = wl.random_normal_f32((256, 300), 22) * np.float32(37.0)
    for fmt in (orc.FMT_E4M3, orc.FMT_E5M2):
        s = orc.scale(orc.amax(x), fmt, pow2=True)
        q = orc.quantize(x, s, fmt)
        enc = orc.e5m2_encode if fmt == orc.FMT_E5M2 else orc.e4m3_encode
        assert np.array_equal(q, enc(x.astype(np.float64) / float(s)))
        # nothing saturates: every |x/s| <= the format maximum
        dec = orc.fp8_decode(q, fmt)
        fmax = 57344.0 if fmt == orc.FMT_E5M2 else 448.0
        assert np.all(np.abs(dec) <= fmax)


# -------------------------------------------------------------------- GEMM

def _exact(Ad, Bd):
    M, K = Ad.shape
    N = Bd.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in Ad]
    Bf = [[Fraction(float(v)) for v in row] for row in Bd]
    R = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    return R, S


random_e5m2_codes = wl.random_e5m2_codes


def test_gemm_mixed_formats_brute_force():
    """E5M2 x E5M2, E4M3 x E5M2 and E5M2 x E4M3 on small sizes against exact
    rational sums: S exactly, R within the sequential double-rounding bound."""
    seed = 0
    for fa, fb in ((orc.FMT_E5M2, orc.FMT_E5M2), (orc.FMT_E4M3, orc.FMT_E5M2), (orc.FMT_E5M2, orc.FMT_E4M3)):
        for (M, N, K) in ((1, 1, 1), (2, 3, 5), (5, 4, 8), (3, 7, 16), (8, 8, 8)):
            seed += 1
            A = random_e5m2_codes((M, K), seed) if fa == orc.FMT_E5M2 else wl.random_e4m3_codes((M, K), seed)
            B = random_e5m2_codes((K, N), 500 + seed) if fb == orc.FMT_E5M2 else wl.random_e4m3_codes((K, N), 500 + seed)
            R, S = orc.gemm(fa, A, B, fmt_b=fb)
            Re, Se = _exact(orc.fp8_decode(A, fa), orc.fp8_decode(B, fb))
            for i in range(M):
                for j in range(N):
                    bound = Fraction(K) * Fraction(2) ** -52 * Se[i][j]
                    assert abs(Fraction(R[i, j]) - Re[i][j]) <= bound, (fa, fb, M, N, K, i, j)
                    assert abs(Fraction(S[i, j]) - Se[i][j]) <= bound, (fa, fb, M, N, K, i, j)


def test_gemm_e5m2_transpose_and_all_ones():
    A = random_e5m2_codes((17, 40), 31)
    B = random_e5m2_codes((40, 23), 32)
    R, _ = orc.gemm(orc.FMT_E5M2, A, B)
    Rt, _ = orc.gemm(orc.FMT_E5M2, B.T.copy(), A.T.copy())
    assert np.allclose(R, Rt.T, rtol=1e-12, atol=0)
    ones = np.full((3, 50), 0x3C, np.uint8)                             # 1.0 in E5M2
    R1, _ = orc.gemm(orc.FMT_E5M2, ones, np.full((50, 4), 0x3C, np.uint8))
    assert np.all(R1 == 50.0)


def test_out_fp8_e5m2_vs_torch():
    g = np.random.default_rng(33)
    V = (g.standard_normal(20000) * 1000.0).astype(np.float32).astype(np.float64)
    s_out = 0.5      # a power of two: V / s_out is exact in FP32, so torch's cast sees the same value
    ours = orc.out_fp8(V, s_out, orc.FMT_E5M2)
    ref = torch.from_numpy((V / s_out).astype(np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    inrange = np.abs(V / s_out) < 61440.0
    assert np.array_equal(ours[inrange], ref[inrange])
    assert np.all(ours[~inrange] & 0x7F == 0x7B)
