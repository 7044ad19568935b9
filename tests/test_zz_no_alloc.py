"""GPU check of gemm_fp8_splitk_noalloc (split-K with the library's own
per-GPU array instead of a workspace) against gemm_fp8_splitk with a
workspace: two calls in a row, the second on a smaller input, every output
element bit-identical (same kernels, same order of the FP32 sums) and within
the oracle's bound; a plan larger than the array is refused before any
launch; a shape that does not split is the plain call."""
import numpy as np
import pytest
import torch

import oracle as orc
import precision_dense_gemm_03_amd as g
import workloads as wl
from parity import check_f32, fp8_dot_allowance

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


def run_pair(M, N, K, seed, out_dtype):
    """(no-alloc result, workspace result, codes A, codes B) for one shape."""
    ca = wl.random_e4m3_codes((M, K), seed)
    cb = wl.random_e4m3_codes((K, N), seed + 1)
    ta, tb = dev(ca), dev(cb)
    sa, sb = scalar(0.125), scalar(0.5)
    s_out = scalar(64.0)
    name, splits, nbytes = g.splitk_plan(g.KIND_FP8, g.OUT_F32 if out_dtype == torch.float32 else g.OUT_E4M3,
                                         M, N, K)
    say(f"no-alloc split-K {M}x{N}x{K} {out_dtype}: {name} splits={splits} workspace={nbytes}")
    assert splits > 1 and 0 < nbytes <= g.gemm_fp8_splitk_noalloc_max_bytes()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    c_ws = torch.empty((M, N), dtype=out_dtype, device=DEV)
    c_na = torch.full((M, N), 7, dtype=out_dtype, device=DEV)
    g.gemm_fp8_splitk(ta, g.FMT_E4M3, tb, g.FMT_E4M3, sa, sb, c_ws, s_out, workspace=ws)
    g.gemm_fp8_splitk_noalloc(ta, g.FMT_E4M3, tb, g.FMT_E4M3, sa, sb, c_na, s_out)
    return host(c_na), host(c_ws), ca, cb


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.uint8], ids=["f32", "e4m3"])
def test_noalloc_matches_workspace_entry_point_twice(out_dtype):
    # first call, then a smaller one: the array keeps the first call's partial
    # sums, which the second must not see
    for (M, N, K, seed) in ((4, 4096, 4096, 11), (3, 1000, 1500, 12)):
        got, ref, ca, cb = run_pair(M, N, K, seed, out_dtype)
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), f"{M}x{N}x{K}"
        if out_dtype == torch.float32:
            R, S = orc.gemm(orc.FMT_E4M3, ca, cb)
            check_f32(got, R, S, 0.125, 0.5, what=f"no-alloc {M}x{N}x{K}", T=fp8_dot_allowance(ca, cb))


def test_noalloc_refuses_plans_beyond_the_array(monkeypatch):
    # 16 ranges of 64 x 8192 FP32 sums need 32 MiB: refused on the host
    monkeypatch.setenv("LIBGEMM_CONFIG", "tile_fp8_64x64x128_w2x2")
    monkeypatch.setenv("LIBGEMM_SPLITS", "16")
    M, N, K = 64, 8192, 4096
    _, splits, nbytes = g.splitk_plan(g.KIND_FP8, g.OUT_F32, M, N, K)
    assert splits == 16 and nbytes > g.gemm_fp8_splitk_noalloc_max_bytes()
    say("no-alloc split-K over the limit")
    a = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    b = torch.zeros((K, N), dtype=torch.uint8, device=DEV)
    c = torch.empty((M, N), dtype=torch.float32, device=DEV)
    with pytest.raises(g.GemmError):
        g.gemm_fp8_splitk_noalloc(a, g.FMT_E4M3, b, g.FMT_E4M3, scalar(1.0), scalar(1.0), c)


def test_noalloc_plain_when_the_plan_does_not_split():
    M, N, K = 300, 520, 640
    assert g.splitk_plan(g.KIND_FP8, g.OUT_F32, M, N, K)[1] == 1
    say("no-alloc split-K, plan without split")
    ca, cb = wl.random_e4m3_codes((M, K), 21), wl.random_e4m3_codes((K, N), 22)
    c1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    c2 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    g.gemm_fp8_splitk_noalloc(dev(ca), g.FMT_E4M3, dev(cb), g.FMT_E4M3, scalar(1.0), scalar(1.0), c1)
    g.gemm_fp8_scaled(dev(ca), dev(cb), scalar(1.0), scalar(1.0), c2)
    assert torch.equal(c1, c2)
