"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Every source is compiled on its own (in parallel) and the objects are linked into
token_dispatch_expert_router_amd/libmoe.so.  The routing file is compiled without
floating-point contraction so the softmax rounds each operation on its own.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ROOT = os.path.dirname(PKG)

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
PER_FILE = {"route.hip": ["-ffp-contract=off"]}
SOURCES = ["api.hip", "route.hip", "rows.hip", "gemm_mfma.hip", "gemm_valu.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the MI355X library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


TILE_MAP_CHECK_SRC = os.path.join(ROOT, "tests", "native", "tile_map_check.hip")
TILE_MAP_CHECK = os.path.join(ROOT, "tests", "native", "tile_map_check")


def build_tile_map_check(out: str = TILE_MAP_CHECK) -> str:
    """Host program of the tests: the grouped GEMM's tile maps (csrc/tile_map.h) compiled
    for the CPU only, to walk launch grids over given segment offsets."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), TILE_MAP_CHECK_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on tile_map_check.hip:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if os.path.exists(TILE_MAP_CHECK_SRC):
        build_tile_map_check()
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
