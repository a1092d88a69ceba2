"""Build libqdiff.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc,
and libqdmeasure.so (the benchmark's measurement kernels, measure/*.hip).

Usage: python -m quantized_diffusion_amd.build [-j JOBS] [-v]
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqdiff.so")
MEASURE_SRC = os.path.join(PKG, "measure")
MEASURE_LIB = os.path.join(PKG, "libqdmeasure.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libqdiff.so")
    return exe


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    _link(sorted(glob.glob(os.path.join(MEASURE_SRC, "*.hip"))), MEASURE_LIB, verbose)
    return LIB


def _link(srcs, lib: str, verbose: bool) -> None:
    """One shared library straight from its sources."""
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-shared", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build of {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.v))
