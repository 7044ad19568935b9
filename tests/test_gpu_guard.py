"""GPU parity for the FP16 dynamic-range guard (gemm_f16_guarded): the scale
and the scaled FP16 operands bit-exact against the oracle, the result within
the F32/F16 bounds of the oracle's (A'B')/s, inputs beyond the FP16 range
that a plain cast turns into inf, and the degenerate and error cases."""
import numpy as np
import pytest
import torch

import oracle as orc
import precision_dense_gemm_03_amd as g
import workloads as wl
from parity import check_f16, check_f32

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


def operands(M, N, K, seed, big):
    a = wl.random_normal_f32((M, K), seed) * np.float32(big)
    b = wl.random_normal_f32((K, N), seed + 1) * np.float32(3.0)
    a.reshape(-1)[:: max(1, a.size // 7)] *= np.float32(20.0)      # a few outliers in A
    return a, b


def workspace_views(ws, M, N, K):
    """The scaled FP16 operands inside the documented workspace layout."""
    off_b = 256 + (M * K * 2 + 255) // 256 * 256
    a16 = ws[256:256 + M * K * 2].view(torch.int16)
    b16 = ws[off_b:off_b + K * N * 2].view(torch.int16)
    return host(a16).view(np.uint16).reshape(M, K), host(b16).view(np.uint16).reshape(K, N)


# (M, N, K, magnitude of A): tile and direct-load shapes with ragged edges, the
# decode shape (streaming kernel), magnitudes that need no scaling (s = 1) and
# ones that put A beyond the FP16 range.
CASES = [(64, 80, 96, 1.0), (300, 272, 200, 4000.0), (129, 4096, 1024, 3000.0), (1, 12288, 4096, 2000.0),
         (513, 784, 130, 1.0e4), (16, 100, 33, 0.5)]


@pytest.mark.parametrize("M,N,K,big", CASES)
def test_guarded_gemm_against_oracle(M, N, K, big):
    say(f"guarded f16 {M}x{N}x{K} |A| ~ {big}")
    a, b = operands(M, N, K, M + N + K, big)
    s_ref = orc.guard_scale(orc.amax(a), orc.amax(b))
    a16_ref, b16_ref = orc.guard_to_f16(a, s_ref), orc.guard_to_f16(b, s_ref)
    R, S = orc.gemm(orc.FMT_F16, a16_ref, b16_ref)
    ta, tb = dev(a), dev(b)
    ws = torch.empty(g.guarded_workspace_size(M, N, K), dtype=torch.uint8, device=DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    _, s = g.gemm_f16_guarded(ta, tb, C, workspace=ws)
    got_s = host(s)[0]
    assert np.float32(got_s).view(np.uint32) == np.float32(s_ref).view(np.uint32), (got_s, s_ref)
    a16, b16 = workspace_views(ws, M, N, K)
    assert np.array_equal(a16, a16_ref) and np.array_equal(b16, b16_ref)
    inv = 1.0 / float(s_ref)
    check_f32(host(C), R, S, inv, 1.0, what=f"guarded f32 {M}x{N}x{K}")
    V = R * inv
    if np.all(np.abs(V) + 1e-5 * S * inv < 65504):
        C16 = torch.empty((M, N), dtype=torch.float16, device=DEV)
        g.gemm_f16_guarded(ta, tb, C16, workspace=ws)
        check_f16(host(C16), R, S, inv, 1.0, what=f"guarded f16 {M}x{N}x{K}")


def test_guard_keeps_out_of_range_inputs_finite():
    """A holds values beyond 65504 (a plain FP16 cast makes them inf and the
    plain FP16 GEMM returns inf/NaN); the guarded call returns the finite
    product, within the FP16 rounding bound of the exact FP32 product."""
    M, N, K = 96, 200, 512
    a = wl.random_normal_f32((M, K), 71)
    a[5, 17] = 2.5e5
    a[40, 300] = -1.2e5
    b = wl.random_normal_f32((K, N), 72)
    say("guard against FP16 overflow")
    C_plain = torch.empty((M, N), dtype=torch.float32, device=DEV)
    g.gemm_f16(dev(a).half(), dev(b).half(), C_plain)
    assert not np.all(np.isfinite(host(C_plain)))
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    _, s = g.gemm_f16_guarded(dev(a), dev(b), C)
    got = host(C).astype(np.float64)
    assert host(s)[0] < 1 and np.all(np.isfinite(got))
    exact = a.astype(np.float64) @ b.astype(np.float64)
    bound = (np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64)) * (2.0 ** -10 + 1e-5)
    assert np.all(np.abs(got - exact) <= bound)


def test_guarded_degenerate_and_errors():
    say("guarded degenerate shapes")
    M, N = 5, 7
    A = torch.empty((M, 0), dtype=torch.float32, device=DEV)
    B = torch.empty((0, N), dtype=torch.float32, device=DEV)
    C = torch.full((M, N), 9.0, dtype=torch.float32, device=DEV)
    _, s = g.gemm_f16_guarded(A, B, C)
    assert np.array_equal(host(C), np.zeros((M, N), np.float32)) and host(s)[0] == 1.0
    a, b = operands(20, 30, 40, 5, 1.0)
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(g.GemmError):
        g.gemm_f16_guarded(dev(a), dev(b), torch.empty((20, 30), device=DEV), workspace=small)
