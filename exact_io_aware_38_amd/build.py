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
# Measurement aid for the benchmark (sustained MFMA rate), kept out of libattn.so.
CALIB_LIB = os.path.join(PKG, "libcalib.so")
CALIB_SOURCES = ["calib.hip"]

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


# Kernels allowed to use per-lane scratch memory (register spills), with the
# reason; every other kernel must compile without any. Names are the mangled
# symbols' distinctive parts.
SCRATCH_ALLOWED = {
    # d = 128 prefill with dropout: two values live across the main loop are
    # stored once before it and reloaded once after
    "fwd_prefill_kernelILi128ENS_7NoTableELb1E": "dropout variant, spill outside the main loop",
}
RESOURCES = os.path.join(BUILD, "kernel_resources.txt")


def _resources(stderr: str):
    """(kernel, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD) from the
    compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in stderr.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        key, _, val = text.partition(":")
        val = val.strip()
        if key == "Function Name":
            cur = {"kernel": val}
            out.append(cur)
        elif cur is not None and key in ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "Occupancy [waves/SIMD]"):
            cur[key.split()[0]] = int(val)
    return out


def _compile(src: str):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = (KERNEL_ONLY if src.endswith(".hip") else []) + PER_SOURCE.get(src, [])
    cmd = [_hipcc(), *COMMON, *extra, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libattn.so (and the
    benchmark's libcalib.so). Returns the path of libattn.so.

    Also writes the per-kernel register, scratch and occupancy figures to
    _build/kernel_resources.txt and fails if a kernel outside SCRATCH_ALLOWED
    spills to scratch memory."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(CALIB_SOURCES), 8)) as ex:
        done = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    objs = [o for o, _ in done[:len(SOURCES)]]
    calib_objs = [o for o, _ in done[len(SOURCES):]]
    res = [k for _, ks in done for k in ks]
    with open(RESOURCES, "w") as f:
        for k in res:
            f.write(f"{k['kernel']} VGPRs={k.get('VGPRs')} AGPRs={k.get('AGPRs')} "
                    f"scratch={k.get('ScratchSize')} waves/SIMD={k.get('Occupancy')}\n")
    bad = [k["kernel"] for k in res if k.get("ScratchSize", 0) > 0
           and not any(a in k["kernel"] for a in SCRATCH_ALLOWED)]
    if bad:
        raise RuntimeError("kernels spill to scratch memory: " + ", ".join(bad))
    for out, o in ((LIB, objs), (CALIB_LIB, calib_objs)):
        tmp = out + ".tmp"
        cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *o, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed for {os.path.basename(out)}:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, out)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
