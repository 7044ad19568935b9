"""GPU parity of the K-major B entry points (B given as Bt[N,K], the layout of a
linear layer's weight): gemm_f16_bt, gemm_fp8_scaled_bt and
quantize_fp8_transposed, through the C-ABI, against the oracle.

The oracle always computes with the row-major B; the GPU receives its
transpose (a numpy copy, no arithmetic). Quantize codes must be bit-exact,
GEMM outputs within the per-element bounds of tests/parity.py. Each test
prints the case it is about to launch.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import precision_dense_gemm_03_amd as g
import workloads as wl
from parity import allowance_for, check_e4m3, check_f16, check_f32, check_fp8, fp8_dot_allowance

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


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


def sample_rows(M, n=24):
    rows = set([0, M - 1, M // 2])
    rows.update(range(0, M, max(1, M // n)))
    return sorted(r for r in rows if 0 <= r < M)


def run_f16_bt(a16, b16, out, a_t=None, bt_t=None):
    M, K = a16.shape
    N = b16.shape[1]
    C = torch.empty((M, N), dtype=torch.float32 if out == g.OUT_F32 else torch.float16, device=DEV)
    g.gemm_f16_bt(dev(a16) if a_t is None else a_t, dev(b16.T) if bt_t is None else bt_t, C)
    return host(C)


def run_fp8_bt(qa, qbt, sa, sb, out, s_out=None):
    M, N = qa.shape[0], qbt.shape[0]
    dt = {g.OUT_F32: torch.float32, g.OUT_F16: torch.float16, g.OUT_E4M3: torch.uint8}[out]
    C = torch.empty((M, N), dtype=dt, device=DEV)
    g.gemm_fp8_scaled_bt(qa, qbt, sa, sb, C, None if s_out is None else scalar(s_out))
    return host(C)


# ------------------------------------------------------- transposed quantize

@pytest.mark.parametrize("rows,cols", [(1, 1), (1, 1000), (1000, 1), (63, 65), (64, 64), (129, 200),
                                       (16, 4), (17, 5), (4096, 4096), (1000, 4100), (4097, 33)])
def test_quantize_transposed_bit_exact(rows, cols):
    say(f"quantize_transposed {rows}x{cols}")
    x = wl.normal_with_outliers_f32((rows, cols), rows * 31 + cols)
    x[0, 0] = np.float32(1e30)
    if x.size > 3:
        x.reshape(-1)[3] = np.float32(-0.0)
    rest = np.abs(x)[np.abs(x) < 1e29]
    s = orc.scale_from_amax(np.float32(rest.max() if rest.size else 1.0))
    q = g.quantize_fp8_transposed(dev(x), scalar(s))
    assert tuple(q.shape) == (cols, rows)
    assert np.array_equal(host(q), orc.quantize(x, s).T)


def test_quantize_transposed_unaligned_and_specials():
    say("quantize_transposed unaligned pointers, NaN, inf")
    x = wl.random_normal_f32((130, 70), 5) * np.float32(100.0)
    x[3, 4], x[100, 69], x[129, 0] = np.nan, np.inf, -np.inf
    s = np.float32(0.25)
    base = dev(np.concatenate([np.zeros(1, np.float32), x.reshape(-1)]))
    xs = base[1:].view(130, 70)                                   # 4 bytes past an aligned start
    qbuf = torch.empty(70 * 130 + 1, dtype=torch.uint8, device=DEV)
    q = qbuf[1:].view(70, 130)                                    # unaligned output
    g.quantize_fp8_transposed(xs, scalar(s), q)
    assert np.array_equal(host(q), orc.quantize(x, s).T)


# ------------------------------------------------------------- FP16 GEMM

def test_gemm_f16_bt_small_sizes():
    say("gemm_f16_bt (M,N,K) in [1..8] x [1..8] x {1,3,8,16}")
    seed = 0
    for M in range(1, 9):
        for N in range(1, 9):
            for K in (1, 3, 8, 16):
                seed += 1
                a16 = wl.random_f16((M, K), 700 + seed)
                b16 = wl.random_f16((K, N), 9000 + seed)
                R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
                check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=f"f16 bt {M}x{N}x{K}")
                check_f16(run_f16_bt(a16, b16, g.OUT_F16), R, S, what=f"f16 bt->f16 {M}x{N}x{K}")


EDGE = [(m, n, k) for m in (1, 4, 8, 9, 63, 65, 129) for (n, k) in ((1000, 1000), (520, 999), (300, 4096))]


@pytest.mark.parametrize("M,N,K", EDGE)
def test_gemm_f16_bt_edges(M, N, K):
    say(f"gemm_f16_bt edge {M}x{N}x{K}")
    a16 = wl.random_f16((M, K), M * 5 + K)
    b16 = wl.random_f16((K, N), N * 7 + K)
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=f"f16 bt {M}x{N}x{K}")
    check_f16(run_f16_bt(a16, b16, g.OUT_F16), R, S, what=f"f16 bt->f16 {M}x{N}x{K}")


def test_gemm_f16_bt_unaligned_operands():
    say("gemm_f16_bt unaligned A and Bt (element loads)")
    M, N, K = 70, 90, 136
    a16 = wl.random_f16((M, K), 1)
    b16 = wl.random_f16((K, N), 2)
    abuf = dev(np.concatenate([np.zeros(1, np.float16), a16.reshape(-1)]))
    bbuf = dev(np.concatenate([np.zeros(1, np.float16), np.ascontiguousarray(b16.T).reshape(-1)]))
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    got = run_f16_bt(a16, b16, g.OUT_F32, a_t=abuf[1:].view(M, K), bt_t=bbuf[1:].view(N, K))
    check_f32(got, R, S, what="f16 bt unaligned")
    for M in (1, 5):
        a1 = a16[:M]
        got = run_f16_bt(a1, b16, g.OUT_F32, a_t=abuf[1:1 + M * K].view(M, K), bt_t=bbuf[1:].view(N, K))
        R1, S1 = orc.gemm(orc.FMT_F16, a1.view(np.uint16), b16.view(np.uint16))
        check_f32(got, R1, S1, what=f"f16 bt decode unaligned M={M}")


def test_gemm_f16_bt_C1():
    w = wl.C1
    say(f"gemm_f16_bt {w.name}")
    a16, b16 = wl.operand(w, 0), wl.operand(w, 1)
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=w.name)


@pytest.mark.parametrize("w", wl.C3, ids=lambda w: w.name)
def test_gemm_f16_bt_decode_C3(w):
    say(f"gemm_f16_bt {w.name}")
    a16, b16 = wl.operand(w, 0), wl.operand(w, 1)
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    check_f16(run_f16_bt(a16, b16, g.OUT_F16), R, S, what=w.name)


@pytest.mark.parametrize("w", [wl.M0, wl.C5_F16], ids=lambda w: w.name)
def test_gemm_f16_bt_large_sampled(w):
    say(f"gemm_f16_bt {w.name}")
    a16, b16 = wl.operand(w, 0), wl.operand(w, 1)
    rows = sample_rows(w.M, 16)
    got = run_f16_bt(a16, b16, g.OUT_F16)[rows]
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16), rows=rows)
    check_f16(got, R, S, what=w.name)


def test_gemm_f16_bt_matches_row_major_tile_bitwise():
    """Same tile configuration, same operand values in the same k order: the
    K-major and row-major 256x256 tile kernels give identical bits."""
    say("gemm_f16_bt vs gemm_f16, 4096^3")
    a = torch.randn(4096, 4096, device=DEV).half()
    b = torch.randn(4096, 4096, device=DEV).half()
    c1 = torch.empty(4096, 4096, device=DEV, dtype=torch.float32)
    c2 = torch.empty_like(c1)
    g.gemm_f16(a, b, c1)
    g.gemm_f16_bt(a, b.t().contiguous(), c2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# -------------------------------------------------------------- FP8 GEMM

def fp8_chain_bt(xa, xb):
    """GPU amax -> scale -> quantize A, and quantize B transposed; codes and
    scales checked bit-exact against the oracle."""
    ta, tb = dev(xa), dev(xb)
    amax_a, s_a = g.amax_f32(ta)
    amax_b, s_b = g.amax_f32(tb)
    qa = g.quantize_fp8(ta, s_a)
    qbt = g.quantize_fp8_transposed(tb, s_b)
    osa, osb = orc.scale_from_amax(orc.amax(xa)), orc.scale_from_amax(orc.amax(xb))
    assert host(s_a)[0] == osa and host(s_b)[0] == osb
    oqa, oqb = orc.quantize(xa, osa), orc.quantize(xb, osb)
    assert np.array_equal(host(qa), oqa)
    assert np.array_equal(host(qbt), oqb.T)
    return qa, s_a, qbt, s_b, oqa, osa, oqb, osb


def test_gemm_fp8_bt_small_sizes():
    say("gemm_fp8_scaled_bt (M,N,K) in [1..8] x [1..8] x {1,5,16,32}")
    seed = 0
    sa, sb = scalar(0.75), scalar(1.5)
    for M in range(1, 9):
        for N in range(1, 9):
            for K in (1, 5, 16, 32):
                seed += 1
                ca = wl.random_e4m3_codes((M, K), 300 + seed)
                cb = wl.random_e4m3_codes((K, N), 8000 + seed)
                R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
                # M <= 8 runs the FP32-FMA decode kernels: the plain bound
                T = allowance_for(g.select_config_bt(g.KIND_FP8, g.OUT_F32, M, N, K), ca, cb)
                check_f32(run_fp8_bt(dev(ca), dev(cb.T), sa, sb, g.OUT_F32), R, S, 0.75, 1.5,
                          what=f"fp8 bt {M}x{N}x{K}", T=T)


@pytest.mark.parametrize("M,N,K", EDGE)
def test_gemm_fp8_bt_edges(M, N, K):
    say(f"gemm_fp8_scaled_bt edge {M}x{N}x{K}")
    ca = wl.random_e4m3_codes((M, K), M * 3 + K)
    cb = wl.random_e4m3_codes((K, N), N * 17 + K)
    sa, sb = np.float32(0.02), np.float32(0.003)
    R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
    T = allowance_for(g.select_config_bt(g.KIND_FP8, g.OUT_F32, M, N, K), ca, cb)
    ta, tbt, tsa, tsb = dev(ca), dev(cb.T), scalar(sa), scalar(sb)
    check_f32(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_F32), R, S, sa, sb, what="f32", T=T)
    check_f16(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_F16), R, S, sa, sb, what="f16", T=T)
    s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(sa) * float(sb)))))
    check_e4m3(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_E4M3, s_out), R, S, sa, sb, s_out, what="e4m3", T=T)


def test_gemm_fp8_bt_C2():
    w = wl.C2
    say(f"gemm_fp8_scaled_bt {w.name}")
    qa, sa, qbt, sb, oqa, osa, oqb, osb = fp8_chain_bt(wl.operand(w, 0), wl.operand(w, 1))
    R, S = orc.gemm(orc.FMT_E4M3, oqa, oqb)
    check_f32(run_fp8_bt(qa, qbt, sa, sb, g.OUT_F32), R, S, osa, osb, what=w.name)


@pytest.mark.parametrize("w", wl.C4, ids=lambda w: w.name)
def test_gemm_fp8_bt_C4_fp8_output(w):
    say(f"gemm_fp8_scaled_bt {w.name}")
    qa, sa, qbt, sb, oqa, osa, oqb, osb = fp8_chain_bt(wl.operand(w, 0), wl.operand(w, 1))
    rows = None if w.M <= 129 else sample_rows(w.M)
    R, S = orc.gemm(orc.FMT_E4M3, oqa, oqb, rows=rows)
    s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(osa) * float(osb)))))
    got = run_fp8_bt(qa, qbt, sa, sb, g.OUT_E4M3, s_out)
    if rows is not None:
        got = got[rows]
    check_e4m3(got, R, S, osa, osb, s_out, what=w.name)


def test_gemm_fp8_bt_C5_sampled():
    w = wl.C5_FP8
    say(f"gemm_fp8_scaled_bt {w.name}")
    qa, sa, qbt, sb, oqa, osa, oqb, osb = fp8_chain_bt(wl.operand(w, 0), wl.operand(w, 1))
    rows = sample_rows(w.M, 16)
    got = run_fp8_bt(qa, qbt, sa, sb, g.OUT_F16)[rows]
    R, S = orc.gemm(orc.FMT_E4M3, oqa, oqb, rows=rows)
    check_f16(got, R, S, osa, osb, what=w.name)


def test_gemm_fp8_bt_4096_against_oracle_and_deterministic():
    """The K-major FP8 tile kernel at 4096^3 on full-range codes: sampled rows
    within the FP32 bound plus the FP8 matrix-core allowance, and two launches
    bit-identical. (It takes each lane's 32 codes as two 16-code pieces of the
    row, A and B alike, so its sum order differs from the row-major kernel's.)"""
    say("gemm_fp8_scaled_bt 4096^3 vs oracle, twice")
    ca = wl.random_e4m3_codes((4096, 4096), 1)
    cb = wl.random_e4m3_codes((4096, 4096), 2)
    ta, tbt, s = dev(ca), dev(cb.T), scalar(0.5)
    outs = []
    for _ in range(2):
        c = torch.empty(4096, 4096, device=DEV, dtype=torch.float32)
        g.gemm_fp8_scaled_bt(ta, tbt, s, s, c)
        outs.append(host(c))
    assert np.array_equal(outs[0], outs[1])
    rows = sample_rows(4096, 12)
    R, S = orc.gemm(orc.FMT_E4M3, ca, cb, rows=rows)
    check_f32(outs[0][rows], R, S, 0.5, 0.5, what="fp8 bt 4096^3", T=fp8_dot_allowance(ca, cb, rows=rows))


# ----------------------------------------- every K-major configuration forced

FP8_BT_CONFIGS = ["pp_fp8_256x256x64_bt", "pp_fp8_192x256x64_bt", "dma_fp8_256x256x64_s4_bt", "tile_fp8_256x256x128_w2x4_bt", "tile_fp8_128x128x128_w2x2_bt",
                  "tile_fp8_64x64x128_w2x2_bt", "ring_fp8_16x16x128_bt", "ring_fp8_32x32x128_bt", "ring_fp8_64x64x128_bt"]
F16_BT_CONFIGS = ["pp_f16_256x256x32_bt", "pp_f16_192x256x32_bt", "dma_f16_256x256x32_s4_bt", "tile_f16_256x256x64_w2x4_bt", "tile_f16_128x128x64_w2x2_bt",
                  "tile_f16_64x64x64_w2x2_bt", "ring_f16_16x16x64_bt", "ring_f16_32x32x64_bt", "ring_f16_64x64x64_bt"]
# full tiles; M/N edges with a K tail; odd K tile counts; a single partial K
# tile; K not a multiple of 16 bytes (element loads / the register-staged kernel)
FP8_BT_SHAPES = [(256, 256, 256), (300, 272, 80), (513, 784, 192), (100, 32, 48), (257, 520, 1088), (130, 200, 100)]
F16_BT_SHAPES = [(256, 256, 256), (300, 272, 80), (513, 784, 200), (100, 32, 24), (257, 520, 544), (130, 204, 100)]


@pytest.mark.parametrize("cfg", FP8_BT_CONFIGS)
def test_fp8_bt_config_parity(cfg, monkeypatch):
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    sa, sb = np.float32(0.02), np.float32(0.003)
    tsa, tsb = scalar(sa), scalar(sb)
    for (M, N, K) in FP8_BT_SHAPES:
        assert g.select_config_bt(g.KIND_FP8, g.OUT_F32, M, N, K) == cfg
        say(f"{cfg} fp8 {M}x{N}x{K}")
        ca = wl.random_e4m3_codes((M, K), 41 * M + K)
        cb = wl.random_e4m3_codes((K, N), 43 * N + K)
        R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
        T = fp8_dot_allowance(ca, cb)
        ta, tbt = dev(ca), dev(cb.T)
        check_f32(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_F32), R, S, sa, sb, what=f"{cfg} f32 {M}x{N}x{K}", T=T)
        check_f16(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_F16), R, S, sa, sb, what=f"{cfg} f16 {M}x{N}x{K}", T=T)
        s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(sa) * float(sb)))))
        check_e4m3(run_fp8_bt(ta, tbt, tsa, tsb, g.OUT_E4M3, s_out), R, S, sa, sb, s_out,
                   what=f"{cfg} e4m3 {M}x{N}x{K}", T=T)


@pytest.mark.parametrize("cfg", F16_BT_CONFIGS)
def test_f16_bt_config_parity(cfg, monkeypatch):
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    for (M, N, K) in F16_BT_SHAPES:
        assert g.select_config_bt(g.KIND_F16, g.OUT_F32, M, N, K) == cfg
        say(f"{cfg} f16 {M}x{N}x{K}")
        a16 = wl.random_f16((M, K), 47 * M + K)
        b16 = wl.random_f16((K, N), 53 * N + K)
        R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
        check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=f"{cfg} f32 {M}x{N}x{K}")
        check_f16(run_f16_bt(a16, b16, g.OUT_F16), R, S, what=f"{cfg} f16 {M}x{N}x{K}")


@pytest.mark.parametrize("kind,family", [("fp8", "dma"), ("f16", "dma"), ("fp8", "pp"), ("f16", "pp"), ("fp8", "pp192"), ("f16", "pp192"), ("fp8", "ring"),
                                         ("f16", "ring")])
def test_dma_bt_matches_row_major_dma_bitwise(kind, family, monkeypatch):
    """The direct-load, ping-pong and deep-ring kernels with K-major B and with
    row-major B feed the same operand values in the same k order to the same
    MFMAs."""
    M, N, K = (1024, 768, 512) if family != "ring" else (200, 768, 2560)
    say(f"{family} {kind} K-major vs row-major, {M} x {N} x {K}")
    if kind == "fp8":
        a = dev(wl.random_e4m3_codes((M, K), 5))
        b = dev(wl.random_e4m3_codes((K, N), 6))
        s = scalar(0.25)
        run = lambda bb, c, bt: (g.gemm_fp8_scaled_bt if bt else g.gemm_fp8_scaled)(a, bb, s, s, c)  # noqa: E731
        names = {"dma": ("dma_fp8_256x256x64_s4", "dma_fp8_256x256x64_s4_bt"),
                 "pp": ("pp_fp8_256x256x64", "pp_fp8_256x256x64_bt"),
                 "pp192": ("pp_fp8_192x256x64", "pp_fp8_192x256x64_bt"),
                 "ring": ("ring_fp8_64x64x128", "ring_fp8_64x64x128_bt")}[family]
    else:
        a = dev(wl.random_f16((M, K), 5))
        b = dev(wl.random_f16((K, N), 6))
        run = lambda bb, c, bt: (g.gemm_f16_bt if bt else g.gemm_f16)(a, bb, c)  # noqa: E731
        names = {"dma": ("dma_f16_256x256x32_s4", "dma_f16_256x256x32_s4_bt"),
                 "pp": ("pp_f16_256x256x32", "pp_f16_256x256x32_bt"),
                 "pp192": ("pp_f16_192x256x32", "pp_f16_192x256x32_bt"),
                 "ring": ("ring_f16_64x64x64", "ring_f16_64x64x64_bt")}[family]
    c1 = torch.empty(M, N, device=DEV, dtype=torch.float32)
    c2 = torch.empty_like(c1)
    monkeypatch.setenv("LIBGEMM_CONFIG", names[0])
    run(b, c1, False)
    monkeypatch.setenv("LIBGEMM_CONFIG", names[1])
    run(b.t().contiguous(), c2, True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ------------------------------------------- every K-major decode configuration

GEMV_CONFIGS = [("gemv_coop_f16_m1_r4_w8", 0, 1), ("gemv_bt_f16_m1_r4_u4", 0, 1), ("gemv_bt_f16_m4_r2_u4", 0, 4),
                ("gemv_bt_f16_m4_r4_u2", 0, 4), ("gemv_coop_f16_m4_r2_w8", 0, 4), ("gemv_bt_f16_m8_r4_u2", 0, 8),
                ("gemv_bt_f16_m8_r2_u2", 0, 8), ("gemv_bt_fp8_m1_r4_u4", 1, 1), ("gemv_bt_fp8_m1_r2_u4", 1, 1), ("gemv_bt_fp8_m1_r1_u4", 1, 1),
                ("gemv_coop_fp8_m1_r4_w4", 1, 1), ("gemv_coop_fp8_m4_r4_w4", 1, 4), ("gemv_bt_fp8_m4_r4_u2", 1, 4),
                ("gemv_coop_fp8_m8_r2_w4", 1, 8), ("gemv_bt_fp8_m8_r2_u2", 1, 8)]


@pytest.mark.parametrize("cfg,kind,bound", GEMV_CONFIGS, ids=[c[0] for c in GEMV_CONFIGS])
def test_gemv_bt_config_parity(cfg, kind, bound, monkeypatch):
    """Each decode configuration forced on ragged shapes: M up to its bound, N
    not a multiple of the rows per workgroup, K with a tail of elements, K not
    16-byte aligned (element path), K longer than one pass of the lanes."""
    monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    ms = sorted({1, max(1, bound - 1), bound})
    ks = (1, 24, 999, 4104) if kind == 0 else (1, 48, 999, 4112)
    seed = 0
    for M in ms:
        for N in (1, 37, 1000):
            for K in ks:
                seed += 1
                assert g.select_config_bt(kind, g.OUT_F32, M, N, K) == cfg
                say(f"{cfg} {M}x{N}x{K}")
                if kind == 0:
                    a16 = wl.random_f16((M, K), 61 * seed)
                    b16 = wl.random_f16((K, N), 67 * seed)
                    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
                    check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=f"{cfg} f32 {M}x{N}x{K}")
                    check_f16(run_f16_bt(a16, b16, g.OUT_F16), R, S, what=f"{cfg} f16 {M}x{N}x{K}")
                else:
                    ca = wl.random_e4m3_codes((M, K), 71 * seed)
                    cb = wl.random_e4m3_codes((K, N), 73 * seed)
                    sa, sb = np.float32(0.02), np.float32(0.003)
                    R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
                    ta, tbt = dev(ca), dev(cb.T)
                    check_f32(run_fp8_bt(ta, tbt, scalar(sa), scalar(sb), g.OUT_F32), R, S, sa, sb,
                              what=f"{cfg} f32 {M}x{N}x{K}")
                    s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(sa) * float(sb)))))
                    check_e4m3(run_fp8_bt(ta, tbt, scalar(sa), scalar(sb), g.OUT_E4M3, s_out), R, S, sa, sb, s_out,
                               what=f"{cfg} e4m3 {M}x{N}x{K}")


# ------------------------------------------------------------ K-major split-K

@pytest.mark.parametrize("M", [9, 63, 65, 129, 256])
def test_fp8_splitk_bt_C4_shapes(M):
    """Split-K over K-major B at the M-sweep shapes (N = K = 4096, E4M3 output
    with its own scale, the sweep's outlier inputs), against the oracle; a
    second call must give the same bits (slices are added in range order)."""
    w = next((x for x in wl.C4 if x.M == M), None)
    xa = wl.operand(w, 0) if w else wl.normal_with_outliers_f32((M, 4096), 900 + M)
    xb = wl.operand(w, 1) if w else wl.normal_with_outliers_f32((4096, 4096), 901)
    say(f"gemm_fp8_splitk_bt M={M}")
    qa, sa, qbt, sb, oqa, osa, oqb, osb = fp8_chain_bt(xa, xb)
    cfg, splits, nbytes = g.splitk_plan_bt(g.KIND_FP8, g.OUT_E4M3, M, 4096, 4096)
    assert cfg.startswith("ring_fp8") and splits == 1, (cfg, splits)   # M <= 256: the deep-ring kernel
    nbytes = max(nbytes, 16)
    R, S = orc.gemm(orc.FMT_E4M3, oqa, oqb)
    s_out = orc.scale_from_amax(np.float32(np.max(np.abs(R * float(osa) * float(osb)))))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(2):
        C = torch.empty((M, 4096), dtype=torch.uint8, device=DEV)
        g.gemm_fp8_splitk_bt(qa, qbt, sa, sb, C, scalar(s_out), workspace=ws)
        outs.append(host(C))
    assert np.array_equal(outs[0], outs[1])
    check_e4m3(outs[0], R, S, osa, osb, s_out, what=f"splitk bt M={M}")
    # F32 output: the x50 outliers put products more than 2^6 apart in one
    # aligned group of 8 k, so the FP8 matrix cores' alignment allowance applies
    # (on sampled rows: the allowance costs O(M N K) host work)
    C = torch.empty((M, 4096), dtype=torch.float32, device=DEV)
    g.gemm_fp8_splitk_bt(qa, qbt, sa, sb, C, workspace=ws)
    rows = sample_rows(M, 8)
    check_f32(host(C)[rows], R[rows], S[rows], osa, osb, what=f"splitk bt f32 M={M}",
              T=fp8_dot_allowance(oqa, oqb, rows=rows))


@pytest.mark.parametrize("M", [9, 16, 64, 100])
def test_f16_splitk_bt_decode_weight(M):
    """Split-K over the K-major FP16 weight [4096,12288] for M past the decode
    kernels' bound, F16 and F32 outputs, against the oracle."""
    say(f"gemm_f16_splitk_bt M={M}")
    a16 = wl.random_normal_f32((M, 4096), 950 + M).astype(np.float16)
    b16 = (wl.random_normal_f32((4096, 12288), 951) * np.float32(0.02)).astype(np.float16)
    cfg, splits, nbytes = g.splitk_plan_bt(g.KIND_F16, g.OUT_F16, M, 12288, 4096)
    assert cfg.startswith("ring_f16") and splits == 1, (cfg, splits)   # M <= 256: the deep-ring kernel
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    ta, tbt = dev(a16), dev(b16.T)
    for out, dt, chk in ((g.OUT_F16, torch.float16, check_f16), (g.OUT_F32, torch.float32, check_f32)):
        C = torch.empty((M, 12288), dtype=dt, device=DEV)
        g.gemm_f16_splitk_bt(ta, tbt, C)
        chk(host(C), R, S, what=f"f16 splitk bt M={M}")


def test_splitk_bt_decode_shapes_do_not_split():
    """M <= 8 with a workspace runs the decode kernel (the plan does not split)."""
    say("gemm_fp8_splitk_bt M=1 with a workspace")
    ca = wl.random_e4m3_codes((1, 4096), 5)
    cb = wl.random_e4m3_codes((4096, 1000), 6)
    assert g.splitk_plan_bt(g.KIND_FP8, g.OUT_F32, 1, 1000, 4096)[1] == 1
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    C = torch.empty((1, 1000), dtype=torch.float32, device=DEV)
    g.gemm_fp8_splitk_bt(dev(ca), dev(cb.T), scalar(1.0), scalar(1.0), C, workspace=ws)
    R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
    check_f32(host(C), R, S, 1.0, 1.0, what="splitk bt decode")


@pytest.mark.parametrize("M,N,K", [(9, 1, 100), (70, 5, 256), (130, 17, 4096), (300, 1, 512)])
def test_tile_bt_narrow_n(M, N, K):
    """K-major tile kernels with fewer output columns than one tile row of B:
    every Bt row past N is clamped to row N-1 and never stored."""
    say(f"tile bt narrow N {M}x{N}x{K}")
    a16 = wl.random_f16((M, K), 3 * M + N)
    b16 = wl.random_f16((K, N), 5 * N + K)
    assert g.select_config_bt(g.KIND_F16, g.OUT_F32, M, N, K).startswith(("tile_", "ring_"))
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    check_f32(run_f16_bt(a16, b16, g.OUT_F32), R, S, what=f"f16 bt {M}x{N}x{K}")
    ca = wl.random_e4m3_codes((M, K), 7 * M + N)
    cb = wl.random_e4m3_codes((K, N), 11 * N + K)
    R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
    check_f32(run_fp8_bt(dev(ca), dev(cb.T), scalar(0.25), scalar(2.0), g.OUT_F32), R, S, 0.25, 2.0,
              what=f"fp8 bt {M}x{N}x{K}", T=fp8_dot_allowance(ca, cb))


# ------------------------------------------------ FP8 operand formats, K-major

ORC_FMT = {g.FMT_E4M3: orc.FMT_E4M3, g.FMT_E5M2: orc.FMT_E5M2}
PAIRS = [(g.FMT_E4M3, g.FMT_E4M3), (g.FMT_E4M3, g.FMT_E5M2), (g.FMT_E5M2, g.FMT_E4M3), (g.FMT_E5M2, g.FMT_E5M2)]
# (config forced, M, N, K): the decode kernels (per-wave M = 1, cooperative
# M <= 4 and M <= 8, by the selector) and each K-major tile configuration
FMT_SHAPES = [(None, 1, 1000, 512), (None, 4, 520, 640), (None, 8, 300, 256),
              ("tile_fp8_64x64x128_w2x2_bt", 100, 200, 256), ("tile_fp8_128x128x128_w2x2_bt", 300, 272, 384),
              ("tile_fp8_256x256x128_w2x4_bt", 257, 512, 320), ("pp_fp8_256x256x64_bt", 300, 272, 192),
              ("ring_fp8_32x64x128_bt", 70, 200, 2048)]


def fp8_codes(fmt, shape, seed):
    return wl.random_e5m2_codes(shape, seed) if fmt == g.FMT_E5M2 else wl.random_e4m3_codes(shape, seed)


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("cfg,M,N,K", FMT_SHAPES)
def test_gemm_fp8_fmt_bt(fa, fb, cfg, M, N, K, monkeypatch):
    if cfg:
        monkeypatch.setenv("LIBGEMM_CONFIG", cfg)
    say(f"gemm_fp8_fmt_bt a={fa} b={fb} {cfg} {M}x{N}x{K}")
    ca = fp8_codes(fa, (M, K), 13 * M + K + fa)
    cb = fp8_codes(fb, (K, N), 17 * N + K + fb)
    ofa, ofb = ORC_FMT[fa], ORC_FMT[fb]
    R, S = orc.gemm(ofa, ca, cb, fmt_b=ofb)
    T = allowance_for(cfg or g.select_config_bt(g.KIND_FP8, g.OUT_F32, M, N, K), ca, cb, fmt_a=ofa, fmt_b=ofb)
    sa, sb = np.float32(0.5), np.float32(0.25)
    ta, tbt, tsa, tsb = dev(ca), dev(cb.T), scalar(sa), scalar(sb)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    g.gemm_fp8_fmt_bt(ta, fa, tbt, fb, tsa, tsb, C)
    check_f32(host(C), R, S, sa, sb, what="f32", T=T)
    V = R * float(sa) * float(sb)
    for out_fmt in (g.FMT_E4M3, g.FMT_E5M2):
        s_out = orc.scale(np.float32(np.max(np.abs(V))), ORC_FMT[out_fmt])
        C = torch.empty((M, N), dtype=torch.uint8, device=DEV)
        g.gemm_fp8_fmt_bt(ta, fa, tbt, fb, tsa, tsb, C, scalar(s_out), out_fmt=out_fmt)
        check_fp8(host(C), R, S, sa, sb, s_out, ORC_FMT[out_fmt], what=f"fp8 out {out_fmt}", T=T)


@pytest.mark.parametrize("rows,cols", [(1, 1), (63, 65), (129, 200), (4096, 1000)])
def test_quantize_transposed_e5m2_bit_exact(rows, cols):
    say(f"quantize_transposed e5m2 {rows}x{cols}")
    x = wl.normal_with_outliers_f32((rows, cols), 77 * rows + cols) * np.float32(1000.0)
    x[0, 0] = np.float32(-1e30)
    for pow2 in (False, True):
        s = orc.scale(orc.amax(x), orc.FMT_E5M2, pow2)
        q = g.quantize_fp8_transposed_fmt(dev(x), scalar(s), g.FMT_E5M2)
        assert np.array_equal(host(q), orc.quantize(x, s, orc.FMT_E5M2).T)


def test_pow2_e5m2_chain_kmajor():
    """FP32 A and B -> power-of-two E5M2 scale for A, E4M3 for B -> quantize A,
    quantize B transposed -> mixed K-major GEMM -> F16; every step against the
    oracle's chain."""
    M, N, K = 300, 1024, 512
    xa = wl.random_normal_f32((M, K), 51) * np.float32(1000.0)
    xb = wl.random_normal_f32((K, N), 52)
    ta, tb = dev(xa), dev(xb)
    _, s_a = g.amax_scale_f32(ta, g.FMT_E5M2, True)
    _, s_b = g.amax_scale_f32(tb, g.FMT_E4M3, True)
    qa = g.quantize_fp8_fmt(ta, s_a, g.FMT_E5M2)
    qbt = g.quantize_fp8_transposed_fmt(tb, s_b, g.FMT_E4M3)
    osa = orc.scale(orc.amax(xa), orc.FMT_E5M2, True)
    osb = orc.scale(orc.amax(xb), orc.FMT_E4M3, True)
    assert host(s_a)[0] == osa and host(s_b)[0] == osb
    cqa, cqb = orc.quantize(xa, osa, orc.FMT_E5M2), orc.quantize(xb, osb, orc.FMT_E4M3)
    assert np.array_equal(host(qa), cqa) and np.array_equal(host(qbt), cqb.T)
    C = torch.empty((M, N), dtype=torch.float16, device=DEV)
    g.gemm_fp8_fmt_bt(qa, g.FMT_E5M2, qbt, g.FMT_E4M3, s_a, s_b, C)
    R, S = orc.gemm(orc.FMT_E5M2, cqa, cqb, fmt_b=orc.FMT_E4M3)
    T = fp8_dot_allowance(cqa, cqb, fmt_a=orc.FMT_E5M2, fmt_b=orc.FMT_E4M3)
    check_f16(host(C), R, S, osa, osb, what="pow2 chain k-major", T=T)


# ------------------------------------------------------------- weight packing

@pytest.mark.parametrize("K,N", [(1, 1), (1, 1000), (1000, 1), (63, 65), (64, 64), (4096, 12288), (4100, 333)])
def test_pack_b_kmajor_exact(K, N):
    """pack_b_kmajor moves FP16 values and FP8 codes unchanged into Bt[N, K]."""
    say(f"pack_b_kmajor {K}x{N}")
    b16 = wl.random_f16((K, N), K + 3 * N)
    bt = g.pack_b_kmajor(dev(b16))
    assert tuple(bt.shape) == (N, K)
    assert np.array_equal(host(bt).view(np.uint16), np.ascontiguousarray(b16.T).view(np.uint16))
    c8 = wl.random_e4m3_codes((K, N), K + 5 * N)
    bt8 = g.pack_b_kmajor(dev(c8))
    assert np.array_equal(host(bt8), np.ascontiguousarray(c8.T))


def test_pack_then_decode():
    """A row-major FP16 weight packed once, then the K-major M = 1 decode, against the oracle."""
    w = wl.C3[0]
    say(f"pack + decode {w.name}")
    a16, b16 = wl.operand(w, 0), wl.operand(w, 1)
    bt = g.pack_b_kmajor(dev(b16))
    C = torch.empty((w.M, w.N), dtype=torch.float16, device=DEV)
    g.gemm_f16_bt(dev(a16), bt, C)
    R, S = orc.gemm(orc.FMT_F16, a16.view(np.uint16), b16.view(np.uint16))
    check_f16(host(C), R, S, what=f"pack + decode {w.name}")
