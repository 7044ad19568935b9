"""Builds libgemm.so (the HIP kernels and the C-ABI) in place, for gfx950 only.

Every source is compiled by hipcc to an object file under _build/, then linked
into precision_dense_gemm_03_amd/libgemm.so. Builds always recompile: this is
the "does it build" check as well as the build.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgemm.so")

SOURCES = ["abi.cpp", "selector.cpp", "amax_quant.hip", "amax_quant_channel.hip", "splitk_reduce.hip",
           "guard_f16.hip", "gemm_tile.hip", "gemm_tile_mixed.hip", "gemm_dma.hip", "gemm_dma_mixed.hip",
           "gemm_stream.hip", "gemv_kmajor.hip", "gemm_pp.hip", "gemm_pp_mixed.hip",
           "amax_quant_pair.hip", "gemm_ring.hip", "gemm_ring_mixed.hip", "noalloc.hip", "gemm_pp_exact.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no packed FP32 VALU instructions (kept off on this target).
# Correctly rounded FP32 divide: the quantizer's x / scale must be IEEE division.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument", "-Wno-inline-asm",
    "-I", CSRC, "-I", INCLUDE,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build_libgemm(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_libgemm(verbose="-v" in sys.argv))
