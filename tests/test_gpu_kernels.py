"""GPU parity per compiled kernel configuration.

The selector sends small problems to small tiles, so the large-tile kernels
would otherwise only meet sampled checks at full size. Here every tile
configuration is forced by name (LIBGEMM_CONFIG) on ragged shapes -- M and N
edges, a K tail, odd and even numbers of K tiles, operands that are not
16-byte aligned (which the direct-load kernel hands to the register-staged
kernel) -- and compared element by element with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import precision_dense_gemm_03_amd as g
import workloads as wl
from parity import check_e4m3, check_f16, check_f32, fp8_dot_allowance

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ORC_FMT_OF = {g.FMT_E4M3: orc.FMT_E4M3, g.FMT_E5M2: orc.FMT_E5M2}


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


def scalar(v):
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=DEV)


FP8_CONFIGS = ["pp_fp8_256x256x64", "pp_fp8_192x256x64", "dma_fp8_256x256x64_s4", "dma_fp8_256x256x64_s5", "tile_fp8_256x256x128_w2x4",
               "tile_fp8_128x128x128_w2x2", "tile_fp8_64x64x128_w2x2", "ring_fp8_16x16x128", "ring_fp8_32x32x128",
               "ring_fp8_64x64x128"]
F16_CONFIGS = ["pp_f16_256x256x32", "pp_f16_192x256x32", "dma_f16_256x256x32_s4", "dma_f16_256x256x32_s5", "tile_f16_256x256x64_w2x4",
               "tile_f16_128x128x64_w2x2", "tile_f16_64x64x64_w2x2", "ring_f16_16x16x64", "ring_f16_32x32x64",
               "ring_f16_64x64x64"]

# (M, N, K): full tiles; M/N edges with a K tail; an odd number of K tiles;
# a single partial K tile; K and N not multiples of 16 bytes (unaligned rows).
FP8_SHAPES = [(256, 256, 256), (300, 272, 80), (513, 784, 192), (100, 32, 48), (257, 512, 1088), (130, 200, 100)]
F16_SHAPES = [(256, 256, 256), (300, 272, 80), (513, 784, 200), (100, 32, 24), (257, 512, 544), (130, 204, 100)]


@pytest.mark.parametrize("cfg", FP8_CONFIGS)
def test_fp8_config_parity(cfg, monkeypatch):
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    sa, sb = np.float32(0.02), np.float32(0.003)
    tsa, tsb = scalar(sa), scalar(sb)
    for (M, N, K) in FP8_SHAPES:
        assert g.select_config(g.KIND_FP8, g.OUT_F32, M, N, K) == cfg
        say(f"{cfg} fp8 {M}x{N}x{K}")
        ca = wl.random_e4m3_codes((M, K), 31 * M + K)
        cb = wl.random_e4m3_codes((K, N), 37 * N + K)
        R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
        T = fp8_dot_allowance(ca, cb)
        ta, tb = dev(ca), dev(cb)
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        g.gemm_fp8_scaled(ta, tb, tsa, tsb, C)
        check_f32(host(C), R, S, sa, sb, what=f"{cfg} f32 {M}x{N}x{K}", T=T)
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        g.gemm_fp8_scaled(ta, tb, tsa, tsb, C)
        check_f16(host(C), R, S, sa, sb, what=f"{cfg} f16 {M}x{N}x{K}", T=T)
        s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(sa) * float(sb)))))
        C = torch.empty((M, N), dtype=torch.uint8, device=DEV)
        g.gemm_fp8_scaled(ta, tb, tsa, tsb, C, scalar(s_out))
        check_e4m3(host(C), R, S, sa, sb, s_out, what=f"{cfg} e4m3 {M}x{N}x{K}", T=T)


@pytest.mark.parametrize("cfg", F16_CONFIGS)
def test_f16_config_parity(cfg, monkeypatch):
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    for (M, N, K) in F16_SHAPES:
        assert g.select_config(g.KIND_F16, g.OUT_F32, M, N, K) == cfg
        say(f"{cfg} f16 {M}x{N}x{K}")
        a16 = wl.random_f16((M, K), 41 * M + K)
        b16 = wl.random_f16((K, N), 43 * N + K)
        R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
        ta, tb = dev(a16), dev(b16)
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        g.gemm_f16(ta, tb, C)
        check_f32(host(C), R, S, what=f"{cfg} f32 {M}x{N}x{K}")
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        g.gemm_f16(ta, tb, C)
        check_f16(host(C), R, S, what=f"{cfg} f16 {M}x{N}x{K}")


RING_CONFIGS = [f"ring_{k}_{bm}x{bn}x{bk}{bt}" for (k, bk) in (("fp8", 128), ("f16", 64))
                for (bm, bn) in ((16, 16), (16, 32), (16, 64), (32, 32), (32, 64), (64, 64)) for bt in ("", "_bt")]
# long K: the unrolled steady loop (at least 15 K tiles), then the tail with a
# partial last tile; M and N edges; a C4 decode-like row block
RING_SHAPES = [(70, 200, 4160), (16, 4096, 4096), (129, 320, 2000), (5, 136, 1936)]


@pytest.mark.parametrize("cfg", RING_CONFIGS)
def test_ring_config_long_k(cfg, monkeypatch):
    """The deep-ring kernel over K long enough to run its unrolled main loop,
    row-major and K-major B, FP8 (F32 and E4M3 outputs) and FP16 operands."""
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    bt = cfg.endswith("_bt")
    for (M, N, K) in RING_SHAPES:
        say(f"{cfg} {M}x{N}x{K}")
        if cfg.startswith("ring_fp8"):
            sel = g.select_config_bt if bt else g.select_config
            assert sel(g.KIND_FP8, g.OUT_F32, M, N, K) == cfg
            ca = wl.random_e4m3_codes((M, K), 61 * M + K)
            cb = wl.random_e4m3_codes((K, N), 67 * N + K)
            R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
            T = fp8_dot_allowance(ca, cb)
            sa, sb = np.float32(0.125), np.float32(0.0625)
            ta, tb = dev(ca), dev(np.ascontiguousarray(cb.T) if bt else cb)
            run = g.gemm_fp8_scaled_bt if bt else g.gemm_fp8_scaled
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            run(ta, tb, scalar(sa), scalar(sb), C)
            check_f32(host(C), R, S, sa, sb, what=f"{cfg} f32 {M}x{N}x{K}", T=T)
            s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(sa) * float(sb)))))
            C = torch.empty((M, N), dtype=torch.uint8, device=DEV)
            run(ta, tb, scalar(sa), scalar(sb), C, scalar(s_out))
            check_e4m3(host(C), R, S, sa, sb, s_out, what=f"{cfg} e4m3 {M}x{N}x{K}", T=T)
        else:
            sel = g.select_config_bt if bt else g.select_config
            assert sel(g.KIND_F16, g.OUT_F32, M, N, K) == cfg
            a16 = wl.random_f16((M, K), 71 * M + K)
            b16 = wl.random_f16((K, N), 73 * N + K)
            R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
            ta, tb = dev(a16), dev(np.ascontiguousarray(b16.T) if bt else b16)
            run = g.gemm_f16_bt if bt else g.gemm_f16
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            run(ta, tb, C)
            check_f32(host(C), R, S, what=f"{cfg} f32 {M}x{N}x{K}")
            C = torch.empty((M, N), dtype=torch.float16, device=DEV)
            run(ta, tb, C)
            check_f16(host(C), R, S, what=f"{cfg} f16 {M}x{N}x{K}")


@pytest.mark.parametrize("kind,cfg", [("fp8", "dma_fp8_256x256x64_s4"), ("f16", "dma_f16_256x256x32_s4"),
                                      ("fp8", "pp_fp8_256x256x64"), ("f16", "pp_f16_256x256x32"),
                                      ("fp8", "pp_fp8_192x256x64"), ("f16", "pp_f16_192x256x32"),
                                      ("fp8", "ring_fp8_32x64x128"), ("f16", "ring_f16_32x64x64")])
def test_direct_load_kernel_offset_operands(kind, cfg, monkeypatch):
    """Operands starting 16 bytes into an allocation (aligned) and 2 bytes in
    (unaligned: handed to the register-staged kernel) give the oracle's result."""
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    M, N, K = 270, 288, 320
    for shift in (16, 2):
        say(f"{cfg} operands shifted by {shift} bytes")
        if kind == "fp8":
            ca = wl.random_e4m3_codes((M, K), 501)
            cb = wl.random_e4m3_codes((K, N), 502)
            ba = torch.zeros(M * K + shift, dtype=torch.uint8, device=DEV)
            bb = torch.zeros(K * N + shift, dtype=torch.uint8, device=DEV)
            ta = ba[shift:].view(M, K)
            tb = bb[shift:].view(K, N)
            ta.copy_(dev(ca))
            tb.copy_(dev(cb))
            R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            g.gemm_fp8_scaled(ta, tb, scalar(1.0), scalar(1.0), C)
            check_f32(host(C), R, S, what=f"fp8 shift {shift}", T=fp8_dot_allowance(ca, cb))
        else:
            a16 = wl.random_f16((M, K), 503)
            b16 = wl.random_f16((K, N), 504)
            ba = torch.zeros(M * K + shift // 2, dtype=torch.float16, device=DEV)
            bb = torch.zeros(K * N + shift // 2, dtype=torch.float16, device=DEV)
            ta = ba[shift // 2:].view(M, K)
            tb = bb[shift // 2:].view(K, N)
            ta.copy_(dev(a16))
            tb.copy_(dev(b16))
            R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            g.gemm_f16(ta, tb, C)
            check_f32(host(C), R, S, what=f"f16 shift {shift}")


# Every streaming (M <= 16) configuration, forced by name: the selector only
# picks some of them by default (M <= 4), the rest stay selectable.
STREAM_CONFIGS = [("stream_f16_m1_c64_t512", 1), ("stream_f16_m1_c64_t1024", 1), ("stream_f16_m1_c64_t256", 1),
                  ("stream_f16_m4_c64_t512", 4), ("stream_f16_m8_c64_t256", 8), ("stream_f16_m16_c64_t256", 16),
                  ("stream_fp8_m1_c64_t1024", 1), ("stream_fp8_m1_c128_t256", 1), ("stream_fp8_m4_c64_t512", 4),
                  ("stream_fp8_m4_c128_t256", 4)]


@pytest.mark.parametrize("cfg,bm", STREAM_CONFIGS)
def test_stream_config_parity(cfg, bm, monkeypatch):
    """Ragged N (not a multiple of the column block), a K tail, every M up to
    the configuration's bound; F32 and F16 (FP8 also E4M3) outputs."""
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    fp8 = "_fp8_" in cfg
    N, K = 1000, 1500
    for M in sorted({1, (bm + 1) // 2, bm}):
        kind = g.KIND_FP8 if fp8 else g.KIND_F16
        assert g.select_config(kind, g.OUT_F32, M, N, K) == cfg
        say(f"{cfg} {M}x{N}x{K}")
        if fp8:
            ca, cb = wl.random_e4m3_codes((M, K), 61 + M), wl.random_e4m3_codes((K, N), 62)
            R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
            ta, tb, one = dev(ca), dev(cb), scalar(1.0)
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            g.gemm_fp8_scaled(ta, tb, one, one, C)
            check_f32(host(C), R, S, what=f"{cfg} f32 M={M}")
            s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R))))
            C8 = torch.empty((M, N), dtype=torch.uint8, device=DEV)
            g.gemm_fp8_scaled(ta, tb, one, one, C8, scalar(s_out))
            check_e4m3(host(C8), R, S, 1.0, 1.0, s_out, what=f"{cfg} e4m3 M={M}")
        else:
            a16, b16 = wl.random_f16((M, K), 63 + M), wl.random_f16((K, N), 64)
            R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
            ta, tb = dev(a16), dev(b16)
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            g.gemm_f16(ta, tb, C)
            check_f32(host(C), R, S, what=f"{cfg} f32 M={M}")
            C16 = torch.empty((M, N), dtype=torch.float16, device=DEV)
            g.gemm_f16(ta, tb, C16)
            check_f16(host(C16), R, S, what=f"{cfg} f16 M={M}")


@pytest.mark.parametrize("cfg", ["pp_fp8_256x256x64", "pp_fp8_192x256x64"])
@pytest.mark.parametrize("bt", [False, True])
def test_pingpong_fp8_out_codes(cfg, bt, monkeypatch):
    """FP8 outputs of the ping-pong kernel on interior tiles, code for code
    against the oracle. The operands are small integers (every product and sum
    is exact in FP32 and on the FP8 matrix cores), so the only rounding is the
    output conversion: ties to even, saturation at the format's largest finite
    value, zeros, and NaN from rows of A that hold the NaN code. Only the waves
    whose rows hold NaN meet one, so both the per-tensor short path and the
    exact code functions it falls back to are exercised in one launch."""
    cfg_bt = cfg + ("_bt" if bt else "")
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg_bt)
    M, N, K = 768, 512, 192       # whole tiles of 256 and of 192 rows; three K tiles
    rng = np.random.default_rng(11)
    ca = orc.e4m3_encode(rng.integers(-12, 13, (M, K)).astype(np.float64))
    cb = orc.e4m3_encode(rng.integers(-12, 13, (K, N)).astype(np.float64))
    for r, k in ((5, 17), (300, 0), (700, 191)):
        ca[r, k] = 0x7F
    R, _ = orc.gemm(orc.FMT_E4M3, ca, cb)
    assert np.isnan(R[[5, 300, 700]]).all() and np.isfinite(np.delete(R, [5, 300, 700], axis=0)).all()
    ta, tb = dev(ca), dev(np.ascontiguousarray(cb.T) if bt else cb)
    one = scalar(1.0)
    for fmt, s_out in ((g.FMT_E4M3, 4.0), (g.FMT_E5M2, 1.0 / 32)):
        ref = orc.out_fp8(R, s_out, ORC_FMT_OF[fmt])
        assert np.any(ref == (0x7E if fmt == g.FMT_E4M3 else 0x7B)), "saturation is covered"
        C = torch.empty((M, N), dtype=torch.uint8, device=DEV)
        say(f"{cfg_bt} fp8 out fmt {fmt} {M}x{N}x{K}")
        call = g.gemm_fp8_scaled_bt if bt else g.gemm_fp8_scaled
        call(ta, tb, one, one, C, scalar(s_out), out_fmt=fmt)
        got = host(C)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{cfg_bt} fmt {fmt}: {len(bad)} codes differ, first at {bad[0]}: " \
                              f"{got[tuple(bad[0])]:#x} vs {ref[tuple(bad[0])]:#x}"


# Long K on the ping-pong kernel: several unrolled 12-step blocks of the main
# loop, then the run-time tail: a partial last K tile, an odd number of full
# tiles (the last A pair holds one tile, loaded with guards), or both; M and N
# edges (clamped rows of A and Bt, clamped columns of row-major B).
# Every shape keeps 16-byte rows (K * e and N * e multiples of 16), so the
# kernel takes it rather than handing it to the register-staged kernel.
PP_LONG = [("pp_fp8_256x256x64", "fp8", (300, 272, 4128)), ("pp_fp8_256x256x64", "fp8", (260, 528, 4160)),
           ("pp_fp8_192x256x64", "fp8", (200, 304, 4208)), ("pp_f16_256x256x32", "f16", (300, 272, 2064)),
           ("pp_f16_192x256x32", "f16", (200, 264, 2080))]


@pytest.mark.parametrize("cfg,kind,shape", PP_LONG)
@pytest.mark.parametrize("bt", [False, True])
def test_pingpong_long_k_tails(cfg, kind, shape, bt, monkeypatch):
    M, N, K = shape
    e = 1 if kind == "fp8" else 2
    assert (K * e) % 16 == 0 and (N * e) % 16 == 0
    name = cfg + ("_bt" if bt else "")
    monkeypatch.setenv("LIBGEMM_CONFIG", name)
    say(f"{name} {M}x{N}x{K}")
    if kind == "fp8":
        ca = wl.random_e4m3_codes((M, K), 3 * M + K)
        cb = wl.random_e4m3_codes((K, N), 5 * N + K)
        R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
        ta, tb = dev(ca), dev(np.ascontiguousarray(cb.T) if bt else cb)
        s1 = scalar(1.0)
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        (g.gemm_fp8_scaled_bt if bt else g.gemm_fp8_scaled)(ta, tb, s1, s1, C)
        check_f32(host(C), R, S, what=name, T=fp8_dot_allowance(ca, cb))
    else:
        a16 = wl.random_f16((M, K), 7 * M + K)
        b16 = wl.random_f16((K, N), 11 * N + K)
        R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
        ta, tb = dev(a16), dev(np.ascontiguousarray(b16.T) if bt else b16)
        C = torch.empty((M, N), dtype=torch.float32, device=DEV)
        (g.gemm_f16_bt if bt else g.gemm_f16)(ta, tb, C)
        check_f32(host(C), R, S, what=name)
