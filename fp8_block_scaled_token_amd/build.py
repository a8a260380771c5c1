"""Build libfp8q.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m fp8_block_scaled_token_amd.build   (or call build()).
Objects go to _build/ at the repository root; the shared library is written
next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8q.so")

SOURCES = ["api.cpp", "quant_kernels.hip", "gemm_kernels.hip", "gemm_fast.hip", "gemm_decode.hip"]

ARCH = "gfx950"

# per-source device code generation options
EXTRA_FLAGS = {
    # MFMA results feed VALU rescale FMAs: keep them in VGPRs, not AGPRs
    "gemm_fast.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gemm_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build fp8q)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        # arithmetic exactly as written: no contraction, IEEE division, denormals kept
        "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-fno-gpu-flush-denormals-to-zero",
        # never emit packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags()
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += EXTRA_FLAGS.get(src, [])
    if save_temps:
        cmd += ["-save-temps=obj"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, save_temps: bool = False) -> str:
    """Compile every source and link libfp8q.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(save_temps="--save-temps" in sys.argv)
