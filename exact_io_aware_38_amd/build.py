"""Ahead-of-time build of libattn.so for gfx950 with hipcc.

Usage: ``python -m exact_io_aware_38_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that the package and the tests load it in-tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["api.cpp", "fwd_bf16.hip", "fwd_f32.hip", "bwd_bf16.hip", "fwd_fp8.hip"]

ARCH = "gfx950"
# Packed fp32 arithmetic is switched off for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]
# Forward kernels: keep MFMA results in ordinary VGPRs instead of shuttling
# them through AGPRs (everything fits in 256 VGPRs, and the softmax reads the
# scores every tile). The backward kernels need more than 256 registers per
# lane; there the accumulators that only MFMAs touch are best left in AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
PER_SOURCE = {"fwd_bf16.hip": VGPR_FORM, "fwd_f32.hip": VGPR_FORM, "fwd_fp8.hip": VGPR_FORM}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


# Kernel sources only: the kernels never produce NaN (masked scores are -inf and
# every -inf - -inf case is guarded), so NaN-preserving max sequences are not
# needed. Host code (argument validation) keeps full IEEE semantics.
KERNEL_ONLY = ["-fno-honor-nans"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = (KERNEL_ONLY if src.endswith(".hip") else []) + PER_SOURCE.get(src, [])
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libattn.so. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
