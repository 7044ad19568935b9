"""amax_quantize_fp8_pair (amax, scale and codes of both GEMM operands in two
launches) against the oracle and against the separate calls, bit for bit."""
import numpy as np
import pytest
import torch

import oracle as orc
import precision_dense_gemm_03_amd as g
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ORC_FMT = {g.FMT_E4M3: orc.FMT_E4M3, g.FMT_E5M2: orc.FMT_E5M2}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(DEV)
    g.lib()
    yield
    torch.cuda.synchronize()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bits(a, b):
    """Bit-identical floats; a NaN matches any NaN (the payload of a
    propagated NaN is not specified)."""
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))


def check_pair(xa, xb, fmt=g.FMT_E4M3, pow2=False, ta=None, tb=None):
    ta = dev(xa) if ta is None else ta
    tb = dev(xb) if (tb is None and xb is not None) else tb
    amax, scale, qa, qb = g.amax_quantize_fp8_pair(ta, tb, fmt=fmt, pow2=pow2)
    ofmt = ORC_FMT[fmt]
    for i, x in enumerate([xa] if xb is None else [xa, xb]):
        oa = orc.amax(x)
        os_ = orc.scale(oa, ofmt, pow2)
        assert same_bits(host(amax)[i], oa), f"amax {i}"
        assert same_bits(host(scale)[i], os_), f"scale {i}"
        q = qa if i == 0 else qb
        assert np.array_equal(host(q).reshape(-1), orc.quantize(x, os_, ofmt).reshape(-1)), f"codes {i}"
    return amax, scale, qa, qb


@pytest.mark.parametrize("w", [wl.C2, wl.C4[2], wl.C4[6]], ids=lambda w: w.name)
def test_pair_workloads(w):
    say(f"pair {w.name}")
    check_pair(wl.operand(w, 0), wl.operand(w, 1))


@pytest.mark.parametrize("na,nb", [(1, 1), (5, 3), (1023, 4097), (1 << 20, 17), (3, 1 << 21), (100003, 0), (0, 77)])
@pytest.mark.parametrize("fmt,pow2", [(g.FMT_E4M3, False), (g.FMT_E5M2, True)])
def test_pair_sizes_formats(na, nb, fmt, pow2):
    say(f"pair sizes {na} {nb} fmt={fmt} pow2={pow2}")
    xa = wl.random_normal_f32((na,), 11 + na) * np.float32(300.0)
    xb = wl.random_normal_f32((nb,), 12 + nb) * np.float32(0.01) if nb else None
    if nb == 0:
        check_pair(xa, None, fmt, pow2)
    else:
        check_pair(xa, xb, fmt, pow2)


def test_pair_random_bit_patterns_and_nan():
    say("pair random bit patterns, NaN")
    rng = np.random.default_rng(5)
    xa = rng.integers(0, 2 ** 32, 1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    xb = wl.random_normal_f32((50000,), 3)
    xb[777] = np.nan
    amax, scale, _, _ = check_pair(xa, xb)
    assert np.isnan(host(amax)[1]) and np.isnan(host(scale)[1])


def test_pair_unaligned_and_matches_separate_calls():
    """Inputs 4 bytes past a 16-byte boundary (scalar paths) and outputs one
    byte in: the same bits as amax_f32 + quantize_fp8 on each tensor."""
    say("pair unaligned")
    xa = wl.random_normal_f32((70001,), 21)
    xb = wl.random_normal_f32((33333,), 22)
    ba, bb = dev(np.concatenate([[0.0], xa]).astype(np.float32)), dev(np.concatenate([[0.0], xb]).astype(np.float32))
    ta, tb = ba[1:], bb[1:]
    qa = torch.empty(xa.size + 1, dtype=torch.uint8, device=DEV)[1:]
    qb = torch.empty(xb.size + 1, dtype=torch.uint8, device=DEV)[1:]
    amax, scale, qa, qb = g.amax_quantize_fp8_pair(ta, tb, qa=qa, qb=qb)
    a1, s1 = g.amax_f32(ta)
    a2, s2 = g.amax_f32(tb)
    q1, q2 = g.quantize_fp8(ta, s1), g.quantize_fp8(tb, s2)
    assert same_bits(host(amax), np.concatenate([host(a1), host(a2)]))
    assert same_bits(host(scale), np.concatenate([host(s1), host(s2)]))
    assert np.array_equal(host(qa), host(q1)) and np.array_equal(host(qb), host(q2))
    check_pair(xa, xb, ta=ta, tb=tb)


def test_pair_then_gemm_chain():
    """The FP8 job of the benchmark: pair quantize, then the GEMM, against the
    oracle's chain (F32 output, sampled rows)."""
    w = wl.C2
    xa, xb = wl.operand(w, 0), wl.operand(w, 1)
    amax, scale, qa, qb = check_pair(xa, xb)
    C = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    g.gemm_fp8_scaled(qa, qb, scale[0:1], scale[1:2], C)
    sa, sb = orc.scale_from_amax(orc.amax(xa)), orc.scale_from_amax(orc.amax(xb))
    R, S = orc.gemm(orc.FMT_E4M3, orc.quantize(xa, sa), orc.quantize(xb, sb))
    from parity import check_f32
    check_f32(host(C), R, S, sa, sb, what="pair chain")


def check_pair_bt(xa, xb, fmt=g.FMT_E4M3, pow2=False, ta=None, tb=None):
    """amax_quantize_fp8_pair_bt against the oracle: the same amax and scales
    as the plain pair, A's codes, and B's codes written transposed."""
    ta = dev(xa) if ta is None else ta
    tb = dev(xb) if tb is None else tb
    amax, scale, qa, qbt = g.amax_quantize_fp8_pair_bt(ta, tb, fmt=fmt, pow2=pow2)
    ofmt = ORC_FMT[fmt]
    K, N = xb.shape
    assert tuple(qbt.shape) == (N, K)
    for i, x in enumerate([xa, xb]):
        oa = orc.amax(x)
        os_ = orc.scale(oa, ofmt, pow2)
        assert same_bits(host(amax)[i], oa), f"amax {i}"
        assert same_bits(host(scale)[i], os_), f"scale {i}"
        ref = orc.quantize(x, os_, ofmt)
        got = host(qa).reshape(x.shape) if i == 0 else host(qbt).T
        assert np.array_equal(got, ref), f"codes {i}: {np.count_nonzero(got != ref)} differ"
    return amax, scale, qa, qbt


# (K, N): whole 128 x 64 blocks with 16-byte rows; ragged edges in both; N
# not a multiple of 4 (element loads); K not a multiple of 16 (element stores);
# a single partial block.
@pytest.mark.parametrize("K,N", [(512, 256), (1000, 777), (130, 68), (256, 66), (48, 20)])
@pytest.mark.parametrize("fmt,pow2", [(g.FMT_E4M3, False), (g.FMT_E5M2, True)])
def test_pair_bt_shapes(K, N, fmt, pow2):
    say(f"pair_bt {K}x{N} fmt {fmt} pow2 {pow2}")
    rng = np.random.default_rng(K * 7 + N)
    xa = (rng.standard_normal((300, 500)) * 3).astype(np.float32)
    xb = (rng.standard_normal((K, N)) * 0.01).astype(np.float32)
    check_pair_bt(xa, xb, fmt, pow2)


def test_pair_bt_special_values_and_offsets():
    """NaN, infinities and values beyond the format's range in B, and A, B and
    the outputs at 4-byte (not 16-byte) offsets."""
    say("pair_bt special values, unaligned")
    rng = np.random.default_rng(5)
    K, N = 384, 192
    xb = (rng.standard_normal((K, N)) * 100).astype(np.float32)
    xb[3, 4], xb[100, 69], xb[129, 0], xb[200, 191] = np.nan, np.inf, -np.inf, 1e30
    xa = rng.standard_normal(4099).astype(np.float32)
    ba = torch.zeros(4099 + 1, dtype=torch.float32, device=DEV)
    bb = torch.zeros(K * N + 1, dtype=torch.float32, device=DEV)
    ta = ba[1:]
    ta.copy_(dev(xa))
    tb = bb[1:].view(K, N)
    tb.copy_(dev(xb))
    amax, scale, qa, qbt = g.amax_quantize_fp8_pair_bt(ta, tb)
    qb = torch.empty((N * K + 4,), dtype=torch.uint8, device=DEV)[4:].view(N, K)
    qa2 = torch.empty((4099 + 4,), dtype=torch.uint8, device=DEV)[4:]
    amax2, scale2, _, _ = g.amax_quantize_fp8_pair_bt(ta, tb, qa=qa2, qbt=qb)
    assert np.isnan(host(amax)[1]) and np.isnan(host(scale)[1])
    # the plain pair on the same inputs: same amax and scales, B's codes transposed
    am_p, sc_p, qa_p, qb_p = g.amax_quantize_fp8_pair(ta, tb)
    assert same_bits(host(amax), host(am_p)) and same_bits(host(scale), host(sc_p))
    assert same_bits(host(amax2), host(am_p)) and same_bits(host(scale2), host(sc_p))
    for q_a, q_b in ((qa, qbt), (qa2, qb)):
        assert np.array_equal(host(q_a), host(qa_p))
        assert np.array_equal(host(q_b), host(qb_p).T)


def test_pair_bt_then_gemm_bt_matches_pair_then_gemm(monkeypatch):
    """The FP8 job both ways: pair + row-major GEMM and pair_bt + K-major GEMM
    on the ping-pong kernel give the same output bits (same codes, same
    scales, and the two layouts' kernels multiply in the same k order)."""
    say("pair_bt + gemm_bt vs pair + gemm, 512 x 768 x 640")
    rng = np.random.default_rng(9)
    M, N, K = 512, 768, 640
    xa = dev(rng.standard_normal((M, K)).astype(np.float32))
    xb = dev((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    _, s1, qa1, qb1 = g.amax_quantize_fp8_pair(xa, xb)
    _, s2, qa2, qbt2 = g.amax_quantize_fp8_pair_bt(xa, xb)
    for out in (torch.float32, torch.float16):
        c1 = torch.empty((M, N), dtype=out, device=DEV)
        c2 = torch.empty((M, N), dtype=out, device=DEV)
        monkeypatch.setenv("LIBGEMM_CONFIG", "pp_fp8_256x256x64")
        g.gemm_fp8_scaled(qa1, qb1, s1[0:1], s1[1:2], c1)
        monkeypatch.setenv("LIBGEMM_CONFIG", "pp_fp8_256x256x64_bt")
        g.gemm_fp8_scaled_bt(qa2, qbt2, s2[0:1], s2[1:2], c2)
        assert torch.equal(c1.view(torch.uint8) if out == torch.float16 else c1.view(torch.int32),
                           c2.view(torch.uint8) if out == torch.float16 else c2.view(torch.int32))
