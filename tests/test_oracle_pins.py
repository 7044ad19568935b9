"""Pins of the oracle to facts outside itself (CPU only).

Each check ties the oracle to the pages' printed values, to closed forms of
the mathematics, or to an independent library routine (torch's float8_e4m3fn
casts, numpy's float16 casts and float64 matmul, Python's exact Fractions),
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_e4m3_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------- E4M3 decode

def test_pages_constants_golden():
    g = json.load(open(GOLDEN))
    dec = orc.e4m3_decode(ALL_CODES)
    finite = dec[~np.isnan(dec)]
    assert finite.max() == g["e4m3_max"]["value"]
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    # 4 exponent bits + 3 mantissa bits: 8 codes per binade above the subnormals
    assert g["e4m3_bits"]["exponent"] == 4 and g["e4m3_bits"]["mantissa"] == 3
    assert dec[0x08] == 2.0 ** -6 and dec[0x10] == 2.0 ** -5
    f16max = orc.f16_decode(np.array([0x7BFF], np.uint16))[0]
    assert f16max == g["f16_max"]["value"]


def test_e4m3_decode_all_256_codes_vs_torch():
    ours = orc.e4m3_decode(ALL_CODES)
    ref = torch_e4m3_decode(ALL_CODES)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # incl. sign of zero


def test_e4m3_decode_structure():
    dec = orc.e4m3_decode(ALL_CODES)
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # strictly increasing 0x00..0x7E
    assert dec[0x01] == 2.0 ** -9                        # min subnormal
    assert dec[0x07] == 7 * 2.0 ** -9                    # max subnormal
    assert np.array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])
    assert np.signbit(dec[0x80]) and dec[0x80] == 0.0


# ----------------------------------------------------------------- E4M3 encode

def test_e4m3_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)


def test_e4m3_encode_midpoints_ties_to_even():
    dec = orc.e4m3_decode(ALL_CODES)
    for c in range(0x7E):
        lo, hi = dec[c], dec[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        got = orc.e4m3_encode(np.array([mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)]))
        assert got[0] == even and got[1] == (0x80 | even)
        assert got[2] == c and got[3] == c + 1


def test_e4m3_encode_special_values():
    v = np.array([-0.0, 0.0, 2.0 ** -10, 1.5 * 2.0 ** -10, -1e-9, 448.0, 456.0, 464.0,
                  464.0001, 1e30, np.inf, -np.inf, -1e30, np.nan, -np.nan, 17.0, 19.0])
    expect = [0x80, 0x00, 0x00, 0x01, 0x80, 0x7E, 0x7E, 0x7E,
              0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x7F, 0x58, 0x5A]
    assert list(orc.e4m3_encode(v)) == expect


def test_e4m3_encode_all_fp32_bit_patterns_vs_torch():
    """All 2^32 FP32 inputs. In [-464, 464] torch's RNE cast is the reference;
    above that torch returns NaN while the pages clamp to +-448 (saturation)."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(chunk, dtype=np.uint32) + np.uint32(start)
        ours = orc.e4m3_encode_f32bits(bits)
        f = bits.view(np.float32)
        with np.errstate(invalid="ignore"):
            absf = np.abs(f)
        nan = np.isnan(f)
        inrange = (~nan) & (absf <= 464.0)
        ref = torch_e4m3_encode_f32(f)
        assert np.array_equal(ours[inrange], ref[inrange]), hex(start)
        big = (~nan) & (absf > 464.0)
        sat = np.where(np.signbit(f[big]), 0xFE, 0x7E).astype(np.uint8)
        assert np.array_equal(ours[big], sat), hex(start)
        assert np.all(ours[nan] == 0x7F), hex(start)


# ----------------------------------------------------------------- FP16 codec

def test_f16_decode_all_codes_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))


def test_f16_round_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    vals = vals[fin]
    nxt = np.nextafter(vals, np.inf)
    g = np.random.default_rng(7)
    cases = [vals,
             (vals[:-1] + vals[1:]) / 2,                       # exact midpoints (ties)
             np.nextafter((vals[:-1] + vals[1:]) / 2, np.inf),
             np.nextafter((vals[:-1] + vals[1:]) / 2, -np.inf),
             g.standard_normal(200000) * 10.0 ** g.uniform(-9, 5, 200000),
             np.array([65504.0, 65519.99, 65520.0, 70000.0, -65520.0, 1e300, np.inf, -np.inf,
                       2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -24, -2.0 ** -26, -0.0])]
    v = np.concatenate(cases)
    ours = orc.f16_round(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    del nxt


# ----------------------------------------------------- amax, scale, quantize

def test_amax_vs_numpy_and_nan():
    x = wl.random_normal_f32((1000, 333), 1)
    x[17, 5] = -9.5
    assert orc.amax(x).view(np.uint32) == np.max(np.abs(x)).view(np.uint32)
    assert orc.amax(x) == np.float32(9.5)
    assert orc.amax(np.zeros(10, np.float32)) == 0.0
    assert orc.amax(np.array([], np.float32)) == 0.0
    y = x.copy()
    y[3, 3] = np.nan
    assert np.isnan(orc.amax(y))
    assert orc.amax(np.array([1.0, -np.inf], np.float32)) == np.inf


def test_scale_from_amax_is_ieee_fp32_division():
    g = np.random.default_rng(3)
    a = np.concatenate([
        (g.random(100000) * 10.0 ** g.uniform(-40, 38, 100000)).astype(np.float32),
        np.frombuffer(g.integers(1, 0x7F800000, 100000, dtype=np.uint32).tobytes(), np.float32)])
    a = a[(a > 0) & np.isfinite(a)]
    with np.errstate(under="ignore"):
        ref = a / np.float32(448.0)            # numpy's IEEE float32 division
    ref = np.where(ref == 0, np.float32(1.0), ref).astype(np.float32)
    ours = np.array([orc.scale_from_amax(x) for x in a[:20000]], np.float32)
    assert np.array_equal(ours.view(np.uint32), ref[:20000].view(np.uint32))
    assert orc.scale_from_amax(0.0) == 1.0
    assert orc.scale_from_amax(np.float32(1e-45)) == 1.0       # underflows to zero -> 1
    assert orc.scale_from_amax(np.float32(448.0)) == 1.0
    assert np.isnan(orc.scale_from_amax(np.float32(np.nan)))


def test_quantize_vs_torch_division_and_cast():
    x = wl.random_normal_f32((512, 513), 5)
    x.reshape(-1)[::97] *= 50.0
    s = orc.scale_from_amax(orc.amax(x))
    q = orc.quantize(x, s)
    t = (torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32))
    ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # the amax element lands on +-448 exactly
    i = np.argmax(np.abs(x))
    assert q.reshape(-1)[i] & 0x7F == 0x7E


def test_quantize_power_of_two_invariance():
    x = wl.random_normal_f32((300, 301), 6)
    s = orc.scale_from_amax(orc.amax(x))
    q0 = orc.quantize(x, s)
    for j in (-20, -3, 1, 7, 30):
        xj = (x * np.float32(2.0 ** j)).astype(np.float32)
        sj = orc.scale_from_amax(orc.amax(xj))
        assert sj == np.float32(s * 2.0 ** j)
        assert np.array_equal(orc.quantize(xj, sj), q0)


def test_quantize_all_ones():
    x = np.ones((4, 8), np.float32)
    s = orc.scale_from_amax(orc.amax(x))
    assert s == np.float32(1.0) / np.float32(448.0)
    assert np.all(orc.quantize(x, s) == 0x7E)


# ------------------------------------------------------------------- GEMM

def _exact_gemm(Ad, Bd):
    M, K = Ad.shape
    N = Bd.shape[1]
    Af = [[Fraction(float(v)) for v in row] for row in Ad]
    Bf = [[Fraction(float(v)) for v in row] for row in Bd]
    R = [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    S = [[sum((abs(Af[i][k] * Bf[k][j]) for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]
    return R, S


def test_gemm_e4m3_brute_force_all_small_sizes():
    """All (M,N,K) in [1..8]^3 over full-range codes: exact rational equality."""
    seed = 0
    for M in range(1, 9):
        for N in range(1, 9):
            for K in range(1, 9):
                seed += 1
                A = wl.random_e4m3_codes((M, K), seed)
                B = wl.random_e4m3_codes((K, N), 10000 + seed)
                R, S = orc.gemm(orc.FMT_E4M3, A, B)
                Re, Se = _exact_gemm(orc.e4m3_decode(A), orc.e4m3_decode(B))
                for i in range(M):
                    for j in range(N):
                        assert Fraction(R[i, j]) == Re[i][j], (M, N, K, i, j)
                        assert Fraction(S[i, j]) == Se[i][j], (M, N, K, i, j)


def test_gemm_f16_brute_force_small_sizes():
    seed = 0
    for M, N, K in [(1, 1, 1), (3, 5, 7), (8, 8, 8), (2, 7, 4), (7, 1, 8), (5, 6, 3)]:
        seed += 1
        A = wl.random_f16((M, K), seed, -100, 100).view(np.uint16)
        B = wl.random_f16((K, N), 100 + seed, -100, 100).view(np.uint16)
        R, S = orc.gemm(orc.FMT_F16, A, B)
        Re, Se = _exact_gemm(orc.f16_decode(A), orc.f16_decode(B))
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(R[i, j]) - Re[i][j])
                assert err <= K * Fraction(2) ** -52 * Se[i][j]
                assert abs(Fraction(S[i, j]) - Se[i][j]) <= K * Fraction(2) ** -52 * Se[i][j]


def test_gemm_e4m3_equals_float64_matmul_exactly():
    A = wl.random_e4m3_codes((1024, 1024), 21)
    B = wl.random_e4m3_codes((1024, 1024), 22)
    R, S = orc.gemm(orc.FMT_E4M3, A, B)
    Ad, Bd = orc.e4m3_decode(A), orc.e4m3_decode(B)
    assert np.array_equal(R, Ad @ Bd)
    assert np.array_equal(S, np.abs(Ad) @ np.abs(Bd))


def test_gemm_identity_and_permutation():
    g = np.random.default_rng(11)
    for fmt, one, A in [(orc.FMT_E4M3, 0x38, wl.random_e4m3_codes((37, 53), 31)),
                        (orc.FMT_F16, 0x3C00, wl.random_f16((37, 53), 32, -50, 50).view(np.uint16))]:
        dec = orc.e4m3_decode if fmt == orc.FMT_E4M3 else orc.f16_decode
        dt = A.dtype
        I = np.zeros((53, 53), dt)
        I[np.arange(53), np.arange(53)] = one
        R, _ = orc.gemm(fmt, A, I)
        assert np.array_equal(R, dec(A))
        perm = g.permutation(37)
        P = np.zeros((37, 37), dt)
        P[np.arange(37), perm] = one
        R, _ = orc.gemm(fmt, P, A)
        assert np.array_equal(R, dec(A)[perm])


def test_gemm_all_ones_gives_K():
    """All-ones operands give C = K (FP8 guide §5.4), also through the quantizer."""
    for M, N, K in [(1, 1, 1), (3, 5, 64), (17, 9, 4096)]:
        R, _ = orc.gemm(orc.FMT_F16, np.full((M, K), 0x3C00, np.uint16), np.full((K, N), 0x3C00, np.uint16))
        assert np.all(R == K)
        x = np.ones((M, K), np.float32)
        y = np.ones((K, N), np.float32)
        sA = orc.scale_from_amax(orc.amax(x))
        sB = orc.scale_from_amax(orc.amax(y))
        R, _ = orc.gemm(orc.FMT_E4M3, orc.quantize(x, sA), orc.quantize(y, sB))
        assert np.all(R == K * 448.0 * 448.0)
        V = R * float(sA) * float(sB)
        assert np.allclose(V, K, rtol=1e-6)


@pytest.mark.parametrize("M", [1, 63, 65, 127, 129])
def test_gemm_edge_sizes_vs_numpy(M):
    K, N = 1024, 1024
    A = wl.random_e4m3_codes((M, K), 100 + M)
    B = wl.random_e4m3_codes((K, N), 200 + M)
    R, _ = orc.gemm(orc.FMT_E4M3, A, B)
    assert np.array_equal(R, orc.e4m3_decode(A) @ orc.e4m3_decode(B))
    Ah = wl.random_f16((M, K), 300 + M).view(np.uint16)
    Bh = wl.random_f16((K, N), 400 + M).view(np.uint16)
    R, S = orc.gemm(orc.FMT_F16, Ah, Bh)
    ref = orc.f16_decode(Ah) @ orc.f16_decode(Bh)
    assert np.all(np.abs(R - ref) <= 4 * K * 2.0 ** -53 * S)


def test_gemm_edge_size_full_depth():
    A = wl.random_e4m3_codes((65, 4096), 501)
    B = wl.random_e4m3_codes((4096, 257), 502)
    R, _ = orc.gemm(orc.FMT_E4M3, A, B)
    assert np.array_equal(R, orc.e4m3_decode(A) @ orc.e4m3_decode(B))


def test_gemm_transpose_and_k_permutation_invariance():
    A = wl.random_e4m3_codes((45, 70), 601)
    B = wl.random_e4m3_codes((70, 33), 602)
    R, S = orc.gemm(orc.FMT_E4M3, A, B)
    Rt, St = orc.gemm(orc.FMT_E4M3, B.T.copy(), A.T.copy())
    assert np.array_equal(R, Rt.T) and np.array_equal(S, St.T)
    perm = np.random.default_rng(5).permutation(70)
    Rp, Sp = orc.gemm(orc.FMT_E4M3, A[:, perm], B[perm, :])
    assert np.array_equal(R, Rp) and np.array_equal(S, Sp)


def test_gemm_row_sampling_matches_full():
    A = wl.random_f16((40, 64), 701).view(np.uint16)
    B = wl.random_f16((64, 24), 702).view(np.uint16)
    R, S = orc.gemm(orc.FMT_F16, A, B)
    rows = [0, 39, 7, 7, 20]
    Rs, Ss = orc.gemm(orc.FMT_F16, A, B, rows=rows)
    assert np.array_equal(Rs, R[rows]) and np.array_equal(Ss, S[rows])


def test_gemm_degenerate_K0():
    R, S = orc.gemm(orc.FMT_E4M3, np.zeros((3, 0), np.uint8), np.zeros((0, 4), np.uint8))
    assert R.shape == (3, 4) and np.all(R == 0) and np.all(S == 0)


# ------------------------------------------------------------ output rounding

def test_out_f16_vs_numpy():
    g = np.random.default_rng(9)
    V = g.standard_normal(100000) * 10.0 ** g.uniform(-8, 5, 100000)
    with np.errstate(over="ignore"):
        ref = V.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.out_f16(V), ref)


def test_out_e4m3_vs_torch_on_fp32_exact_values():
    g = np.random.default_rng(10)
    V = (g.standard_normal(100000) * 10.0 ** g.uniform(-4, 3, 100000)).astype(np.float32)
    s_out = np.float32(0.25)   # a power of two: every quotient below is exactly an FP32 value
    w = (V.astype(np.float64) / np.float64(s_out))
    w32 = w.astype(np.float32)
    exact = w32.astype(np.float64) == w
    ours = orc.out_e4m3(V.astype(np.float64), float(s_out))
    ref = torch_e4m3_encode_f32(w32)
    keep = exact & (np.abs(w32) <= 464)
    assert keep.sum() > 80000
    assert np.array_equal(ours[keep], ref[keep])
    # and the double path agrees with the FP32-bits path whenever w is exactly a float
    assert np.array_equal(ours[exact], orc.e4m3_encode_f32bits(w32[exact].view(np.uint32)))
