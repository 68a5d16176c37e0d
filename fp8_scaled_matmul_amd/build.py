"""Build the HIP library libfp8mi.so in-tree for gfx950 with hipcc.

Usage: python -m fp8_scaled_matmul_amd.build   (or call build()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8mi.so")

SOURCES = ["quantize.hip", "gemm.hip", "gemm_persistent.hip", "gemm_astat.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # bit-exact quantization: no FMA contraction behind the source's back
    "-ffp-contract=off",
    # packed fp32 VALU ops stay off (v_pk_{add,mul,fma}_f32 are never emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file extras.  The block-scaled GEMM promotes each MFMA result on the
# VALU: MFMA results written straight to VGPRs save a copy out of AGPRs.
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the A-stationary kernel's unit loop must unroll fully (its register
         # rings are indexed by the step)
         "gemm_astat.hip": ["-mllvm", "-pragma-unroll-threshold=1000000"]}


def _compile(src: str) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libfp8mi.so (always rebuilds)."""
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
