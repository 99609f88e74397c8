#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step is one pass of the whole training path over one batch of synthetic
input: attn_fwd then attn_bwd on B=1, H=32, S=8192, d=128, causal, bf16 (the
training workload). The same run also times the long-context causal forward
(B=2, H=32, S=8192, d=128, 1% of query rows x30) and the grouped-query decode
(B=16, Hq=32, Hkv=8, one query row against 32768 keys) and a packed batch of
16 causal sequences of 512..3584 tokens (forward + backward through the
variable-length entry points) and the long-context forward on MXFP8 operands
(attn_fwd_fp8 on inputs quantised beforehand; the quantisers are timed on
their own) and the decode on MXFP8 operands, which report as their own sub-objects. Inputs are resident in
device memory before timing starts.

Further sub-objects time the forward alone on the other specified
workloads: the single-head fp32 problem, the four multi-head d=64 variants
(non-causal, causal, ragged keys, ragged causal; with the causal/non-causal
time ratios) and the grouped-query prefill. Every timed entry reports the mean
over the timed steps and the spread of the per-step times (median, p10, p90,
min, max).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibration          (a plain copy of known size,
                                                    for counter calibration)
       python bench.py --only coissue              (matrix pipe and vector ALU shared
                                                    by two wavefronts of one SIMD)
       python bench.py --only mfma_ceiling         (the chip's sustained bf16 MFMA
                                                    rate on an MFMA-only loop)
       python bench.py --summarize-counters WORKLOAD FETCH_DIR WRITE_DIR
                       COPY_FETCH_DIR COPY_WRITE_DIR   (turn rocprofv3 --pmc
                       output into per-kernel HBM-traffic summaries in profiles/)
       python bench.py --summarize-pmc WORKLOAD TITLE DIR [DIR ...]
                       (per-kernel shader counters of rocprofv3 --pmc runs,
                       with MFMA utilisation and instruction mix, in profiles/)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s fwd & fwd+bwd, bf16 d=128 causal S=8K; % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector, published
N_SIMD = 1024                 # 256 CUs x 4 SIMDs
N_XCD = 8
CSRC = os.path.join(ROOT, "exact_io_aware_38_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# kernel name -> source files whose content defines it (for counter staleness)
KERNEL_SOURCES = {
    "fwd_prefill_bf16": ["fwd_bf16.hip", "common.h", "kernels.h", "tiles.h"],
    "fwd_split_bf16": ["fwd_bf16.hip", "common.h", "kernels.h", "tiles.h"],
    "bwd_dkdv": ["bwd_bf16.hip", "common.h", "kernels.h", "tiles.h"],
    "bwd_dkdvq": ["bwd_bf16.hip", "common.h", "kernels.h", "tiles.h"],
    "dq_convert": ["bwd_bf16.hip", "common.h", "kernels.h"],
    "bwd_dq": ["bwd_bf16.hip", "common.h", "kernels.h", "tiles.h"],
    "bwd_pre": ["bwd_bf16.hip", "common.h", "kernels.h"],
    "fwd_fp8": ["fwd_fp8.hip", "common.h", "kernels.h", "tiles.h"],
    "fwd_fp8_split": ["fwd_fp8.hip", "common.h", "kernels.h", "tiles.h"],
    "fwd_f32": ["fwd_f32.hip", "common.h", "kernels.h"],
}
# substrings of the (demangled) device kernel names, as rocprofv3 reports them
# (the dense and the packed instantiations both match; a workload uses one).
# The dK/dV kernel's last template argument tells the fused form (dQ added
# atomically, "bwd_dkdvq") from the two-pass one.
KERNEL_SYMBOLS = {
    "fwd_prefill_bf16": "fwd_prefill_kernel<128,",
    "fwd_split_bf16": "fwd_split_kernel<128>",
    "bwd_dkdv": "bwd_dkdv_kernel<128,",
    "bwd_dkdvq": "bwd_dkdv_kernel<128,",
    "bwd_dq": "bwd_dq_kernel<128,",
    "bwd_pre": "bwd_pre_kernel<128,",
    "dq_convert": "dq_convert_kernel<128>",
    "fwd_fp8": "fwd_fp8_kernel<128>",
    "fwd_fp8_split": "fwd_fp8_split_kernel<128>",
}


def kernel_matches(kernel: str, name: str) -> bool:
    """Whether a demangled rocprofv3 kernel name is an instance of `kernel`."""
    name = _short_kernel_name(name)
    if KERNEL_SYMBOLS[kernel] not in name:
        return False
    if kernel in ("bwd_dkdv", "bwd_dkdvq"):
        return name.replace(" ", "").endswith("true>") == (kernel == "bwd_dkdvq")
    return True


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that an
    edit of comments alone does not mark stored counters as stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str) -> str:
    """Hash of the code (comments and layout ignored) of the files that define
    a kernel; stored with its counters, which bench reports only while it
    still matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def nominal_fwd_flops(B, Hq, Sq, Sk, d, causal) -> float:
    f = 4.0 * B * Hq * Sq * Sk * d
    return f / 2 if causal else f


def kernel_work(kernel: str, w, fused: bool = False) -> dict:
    """Algorithmic work one launch of `kernel` does on workload w.

    Forward: 4*d FLOP per visible (query, key) pair, causal counted as half of
    the pairs. Backward: 10*d per pair over five GEMMs (S recompute, dV, dP, dK,
    dQ); the fused dK/dV/dQ kernel does all five, the two-pass form's dK/dV
    kernel four of them (8*d) and its dQ kernel is credited only with dQ (2*d)
    since its S and dP are a second recomputation. Decode, the preprocess pass
    (which on the fused path also clears the float32 dQ sums) and the dQ
    conversion are bound by bytes: each tensor crosses HBM once.
    """
    fwd = nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    e = 2  # bf16 bytes
    if kernel == "fwd_prefill_bf16":
        return {"bound": "mfma", "flops": fwd}
    if kernel == "fwd_f32":
        return {"bound": "alu", "flops": fwd, "peak": PEAK_F32_VALU_TFLOPS}
    if kernel == "fwd_fp8":
        return {"bound": "mfma", "flops": fwd, "peak": PEAK_FP8_TFLOPS}
    if kernel == "bwd_dkdv":
        return {"bound": "mfma", "flops": 2.0 * fwd}
    if kernel == "bwd_dkdvq":
        return {"bound": "mfma", "flops": 2.5 * fwd}
    if kernel == "dq_convert":
        rows = w.B * w.Hq * w.Sq
        return {"bound": "hbm", "bytes": rows * w.d * (4.0 + e)}
    if kernel == "bwd_dq":
        return {"bound": "mfma", "flops": 0.5 * fwd}
    if kernel == "bwd_pre":
        rows = w.B * w.Hq * w.Sq
        return {"bound": "hbm", "bytes": 2.0 * rows * w.d * e + 3.0 * rows * 4 + (rows * w.d * 4.0 if fused else 0)}
    if kernel == "fwd_split_bf16":
        kv = 2.0 * w.B * w.Hkv * w.Sk * w.d * e
        return {"bound": "hbm", "bytes": kv + w.B * w.Hq * w.Sq * w.d * e}
    if kernel == "fwd_fp8_split":
        kv = 2.0 * w.B * w.Hkv * w.Sk * w.d * (1 + 1 / 32)       # E4M3 codes + one scale byte per 32
        return {"bound": "hbm", "bytes": kv + w.B * w.Hq * w.Sq * w.d * (1 + 1 / 32)}
    if kernel == "combine_split":
        return {"bound": "hbm", "bytes": w.B * w.Hq * w.Sq * (w.d * e + 4)}
    return {"bound": "mfma", "flops": 0.0}


def counters_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"counters_{kernel}__{workload}.json")


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from stored counters, or None if absent or stale."""
    path = counters_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha") != source_hash(kernel):
        return None
    return c.get("hbm_bytes_per_launch")


def roofline(kernel: str, w, avg_ms: float, work: dict = None) -> dict:
    work = kernel_work(kernel, w) if work is None else work
    if work["bound"] in ("mfma", "alu"):
        ach = work["flops"] / (avg_ms * 1e-3) / 1e12
        peak, unit = work.get("peak", PEAK_BF16_TFLOPS), "TFLOP/s"
    else:
        ach = work["bytes"] / (avg_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    return {"kernel": kernel, "bound": work["bound"], "achieved": round(ach, 2), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic_for(kernel, w.name),
            "avg_launch_ms": round(avg_ms, 4)}


def _device_inputs(w):
    import numpy as np
    import torch
    import synth
    x = synth.make_inputs(w)
    out = {}
    for n in ("q", "k", "v", "do"):
        if n in x:
            if w.dtype == "bf16":
                out[n] = torch.from_numpy(x[n].view(np.int16)).cuda().view(torch.bfloat16)
            else:
                out[n] = torch.from_numpy(np.ascontiguousarray(x[n], dtype=np.float32)).cuda()
    del x
    return out


def spread(per_step_ms) -> dict:
    """Median, p10, p90, min and max of the per-step times (ms)."""
    import numpy as np
    a = np.asarray(per_step_ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "min_ms": round(float(a.min()), 4),
            "max_ms": round(float(a.max()), 4), "n": int(a.size)}


def _fwd_workspace(attn, w):
    import torch
    n = attn.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, attn.ATTN_BF16)
    return torch.empty(max(1, n), dtype=torch.uint8, device="cuda")


_LAST_SPREAD = {}


def _time(fn, steps: int, warmup: int, attn, per_step: bool = False):
    """Mean ms per step from events around the timed loop, and each kernel's
    device time: mean per launch, or (per_step) summed over a step. An event
    recorded after every step also gives each step's own time; their spread
    is left in _LAST_SPREAD."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    attn.timing_start()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    kern = attn.timing_stop()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    _LAST_SPREAD.clear()
    _LAST_SPREAD.update(spread([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    if per_step:
        return ms, {k: v[1] / steps for k, v in kern.items()}
    return ms, {k: v[1] / v[0] for k, v in kern.items()}


def bench_step(attn, steps, warmup, fused: bool = False):
    import torch
    import synth
    w = synth.get_workload("train_causal_d128")
    t = _device_inputs(w)
    o = torch.empty_like(t["q"])
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    wsq = attn.bwd_fused_workspace_bytes if fused else attn.bwd_workspace_bytes
    ws = torch.empty(max(1, wsq(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, attn.ATTN_BF16)), dtype=torch.uint8,
                     device="cuda")
    fws = _fwd_workspace(attn, w)

    def step():
        attn.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=fws)
        attn.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, scale=w.scale,
                 dq=dq, dk=dk, dv=dv, workspace=ws, fused=fused)

    ms, kern = _time(step, steps, warmup, attn)
    fwd = nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    total = 3.5 * fwd
    dom = max(kern, key=kern.get)
    return w, ms, total, kern, dom, dict(_LAST_SPREAD)


def bench_fwd(attn, steps, warmup, name: str = "long_causal_d128"):
    """attn_fwd alone on one of the specified workloads (inputs resident)."""
    import torch
    import synth
    w = synth.get_workload(name)
    t = _device_inputs(w)
    o = torch.empty_like(t["q"])
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    fws = _fwd_workspace(attn, w)
    ms, kern = _time(lambda: attn.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, out=o,
                                      lse=lse, workspace=fws), steps, warmup, attn)
    sp = dict(_LAST_SPREAD)
    flops = nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    dom = max(kern, key=kern.get)
    peak = PEAK_F32_VALU_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    return {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk, "d": w.d,
            "causal": w.causal, "dtype": w.dtype, "ms": round(ms, 4), "spread": sp,
            "tflops": round(flops / ms / 1e9, 2), "frac_of_peak": round(flops / ms / 1e9 / peak, 4),
            "roofline": roofline(dom, w, kern[dom]),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()}}


# the four multi-head d = 64 variants: non-causal, causal, ragged keys, ragged causal
C2_VARIANTS = {"noncausal": "multihead_d64", "causal": "multihead_d64_causal",
               "ragged": "multihead_d64_ragged", "ragged_causal": "multihead_d64_ragged_causal"}


def bench_multihead_d64(attn, steps, warmup):
    """The four d = 64 prefill variants and the causal/non-causal time ratios
    (skipping the tiles above the diagonal should make causal about twice as
    fast at the same shape)."""
    import torch
    out = {}
    for key, name in C2_VARIANTS.items():
        out[key] = bench_fwd(attn, steps, warmup, name)
        torch.cuda.empty_cache()
    out["noncausal_over_causal_time"] = round(out["noncausal"]["ms"] / out["causal"]["ms"], 3)
    out["ragged_noncausal_over_causal_time"] = round(out["ragged"]["ms"] / out["ragged_causal"]["ms"], 3)
    return out


def bench_fp8(attn, steps, warmup):
    """The long-context forward on MXFP8 operands: the inputs are quantised
    once before timing (as FP8 attention takes FP8 operands); the timed step
    is attn_fwd_fp8 alone. The quantisers are timed separately."""
    import torch
    import synth
    w = synth.get_workload("long_causal_d128")
    t = _device_inputs(w)
    q8, qs = attn.mxfp8_quantize_rows(t["q"])
    k8, ks = attn.mxfp8_quantize_rows(t["k"])
    vt8, vts = attn.mxfp8_quantize_vt(t["v"])
    o = torch.empty_like(t["q"])
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    ms, kern = _time(lambda: attn.fwd_fp8(q8, qs, k8, ks, vt8, vts, causal=w.causal, scale=w.scale, out=o,
                                          lse=lse), steps, warmup, attn)
    sp = dict(_LAST_SPREAD)

    def quant():
        attn.mxfp8_quantize_rows(t["q"], codes=q8, scales=qs)
        attn.mxfp8_quantize_rows(t["k"], codes=k8, scales=ks)
        attn.mxfp8_quantize_vt(t["v"])

    qms, qkern = _time(quant, max(3, steps // 4), 1, attn)
    flops = nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    return {"workload": w.name + "_mxfp8", "B": w.B, "H": w.Hq, "S": w.Sq, "d": w.d, "causal": w.causal,
            "dtype": "e4m3 (MXFP8 operands), fp32 accumulation", "ms": round(ms, 4), "spread": sp,
            "tflops": round(flops / ms / 1e9, 2),
            "frac_of_fp8_peak": round(flops / ms / 1e9 / PEAK_FP8_TFLOPS, 4),
            "frac_of_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "roofline": roofline("fwd_fp8", w.with_(name=w.name + "_mxfp8"), kern["fwd_fp8"]),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
            "quantise_ms": round(qms, 4), "quantise_kernels_ms": {k: round(v, 4) for k, v in qkern.items()},
            # from bf16 operands: quantising Q, K and V, then the FP8 forward
            "with_quantise": {"ms": round(ms + qms, 4), "tflops": round(flops / (ms + qms) / 1e9, 2),
                              "frac_of_bf16_peak": round(flops / (ms + qms) / 1e9 / PEAK_BF16_TFLOPS, 4)}}


def bench_fp8_decode(attn, steps, warmup):
    """The GQA decode on MXFP8 operands (quantised before timing): K and V
    cross HBM as E4M3 codes plus one scale byte per 32 values."""
    import torch
    import synth
    w = synth.get_workload("gqa_decode")
    t = _device_inputs(w)
    ops = attn.mxfp8_quantize_rows(t["q"]) + attn.mxfp8_quantize_rows(t["k"]) + attn.mxfp8_quantize_vt(t["v"])
    del t
    o = torch.empty(w.B, w.Hq, w.Sq, w.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, attn.fwd_fp8_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal)),
                     dtype=torch.uint8, device="cuda")
    ms, kern = _time(lambda: attn.fwd_fp8(*ops, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws),
                     steps, warmup, attn)
    sp = dict(_LAST_SPREAD)
    alg = kernel_work("fwd_fp8_split", w)["bytes"] + w.B * w.Hq * w.Sq * (w.d * 2 + 4)
    return {"workload": w.name + "_mxfp8", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk, "d": w.d,
            "ms": round(ms, 4), "spread": sp, "algorithmic_bytes": int(alg), "gbs": round(alg / ms / 1e6, 1),
            "frac_of_peak": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4),
            "roofline": roofline("fwd_fp8_split", w.with_(name=w.name + "_mxfp8"), kern["fwd_fp8_split"]),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()}}


def bench_decode(attn, steps, warmup):
    import torch
    import synth
    w = synth.get_workload("gqa_decode")
    t = _device_inputs(w)
    o = torch.empty_like(t["q"])
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    ws = torch.empty(attn.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal, attn.ATTN_BF16),
                     dtype=torch.uint8, device="cuda")
    ms, kern = _time(lambda: attn.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, out=o,
                                      lse=lse, workspace=ws), steps, warmup, attn)
    sp = dict(_LAST_SPREAD)
    e = 2
    alg = 2 * w.B * w.Hkv * w.Sk * w.d * e + 2 * w.B * w.Hq * w.Sq * w.d * e + w.B * w.Hq * w.Sq * 4
    return {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk, "d": w.d,
            "ms": round(ms, 4), "spread": sp, "algorithmic_bytes": alg, "gbs": round(alg / ms / 1e6, 1),
            "frac_of_peak": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4),
            "roofline": roofline("fwd_split_bf16", w, kern["fwd_split_bf16"]),
            "kernels_ms": {k: round(v, 4) for k, v in kern.items()}}


def bench_varlen(attn, steps, warmup):
    """Forward + backward over a packed batch of causal sequences of mixed
    lengths, credited with the same nominal work as the dense step, summed
    over the sequences."""
    import numpy as np
    import torch
    import synth
    w = synth.VARLEN_WORKLOADS["varlen_mix_causal_d128"]
    x = synth.make_varlen_inputs(w)
    t = {n: torch.from_numpy(x[n].view(np.int16)).cuda().view(torch.bfloat16) for n in ("q", "k", "v", "do")}
    cq, ck = x["cu_seqlens_q"].tolist(), x["cu_seqlens_k"].tolist()
    del x
    lens = [b - a for a, b in zip(cq, cq[1:])]
    o = torch.empty_like(t["q"])
    lse = torch.empty(w.Hq, cq[-1], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    nb = attn.bwd_varlen_workspace_bytes(cq, ck, w.Hq, w.Hkv, w.d, w.causal, attn.ATTN_BF16)
    nf = attn.fwd_varlen_workspace_bytes(cq, ck, w.Hq, w.Hkv, w.d, w.causal, attn.ATTN_BF16)
    ws = torch.empty(max(1, nb, nf), dtype=torch.uint8, device="cuda")

    def step():
        attn.fwd_varlen(t["q"], t["k"], t["v"], cq, ck, causal=w.causal, scale=w.scale, out=o, lse=lse,
                        workspace=ws)
        attn.bwd_varlen(t["q"], t["k"], t["v"], o, lse, t["do"], cq, ck, causal=w.causal, scale=w.scale,
                        dq=dq, dk=dk, dv=dv, workspace=ws)

    ms, kern = _time(step, steps, warmup, attn, per_step=True)
    sp = dict(_LAST_SPREAD)
    total = sum(3.5 * nominal_fwd_flops(1, w.Hq, n, n, w.d, w.causal) for n in lens)
    # every kernel runs once per step (at most 64 sequences per launch), so its
    # time per step is its time per launch; the work is summed over sequences
    assert len(lens) <= 64
    dom = max(kern, key=kern.get)
    seq_w = [synth.Workload(w.name, 1, w.Hq, w.Hkv, n, n, w.d, w.dtype, w.causal, seed=0) for n in lens]
    parts = [kernel_work(dom, sw) for sw in seq_w]
    key = "flops" if parts[0]["bound"] == "mfma" else "bytes"
    work = {"bound": parts[0]["bound"], key: sum(p[key] for p in parts)}
    ws_name = w.name
    return {"workload": w.name, "sequences": len(lens), "total_tokens": cq[-1], "min_len": min(lens),
            "max_len": max(lens), "H": w.Hq, "d": w.d, "causal": w.causal,
            "step": "attn_fwd_varlen + attn_bwd_varlen", "ms": round(ms, 4), "spread": sp,
            "tokens_per_s": round(cq[-1] / ms * 1e3, 1), "tflops": round(total / ms / 1e9, 2),
            "frac_of_peak": round(total / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "roofline": roofline(dom, synth.Workload(ws_name, 1, w.Hq, w.Hkv, 0, 0, w.d, w.dtype, w.causal, 0),
                                 kern[dom], work),
            "kernels_ms_per_step": {k: round(v, 4) for k, v in kern.items()}}


def host_description() -> dict:
    """What the CPU baseline ran on: model, logical CPUs, the CPUs this process
    may use, and the BLAS threads the oracle's matrix products use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity": affinity, "blas_threads": blas}


def cpu_baseline(w, heads: int = 8) -> dict:
    """The FP64 oracle as it stands, on a bounded sample of each measured
    workload: fwd + bwd on a few heads of the training workload (the headline
    figure), the forward on one head of the long-context workload, and the
    whole grouped-query decode."""
    import numpy as np
    import oracle
    import synth
    host = host_description()
    x = synth.make_inputs(w)
    f = {n: synth.to_f64(x[n][:, :heads], "bf16") for n in ("q", "k", "v", "do")}
    del x
    t0 = time.perf_counter()
    oracle.attention_forward(f["q"], f["k"], f["v"], causal=w.causal, scale=w.scale)
    oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal=w.causal, scale=w.scale)
    dt = time.perf_counter() - t0
    del f
    flops = 3.5 * nominal_fwd_flops(w.B, heads, w.Sq, w.Sk, w.d, w.causal)
    extra = {}
    # long-context forward: one head (its x30 rows included)
    lw = synth.get_workload("long_causal_d128")
    x = synth.make_inputs(lw)
    f = {n: synth.to_f64(x[n][:1, :1], "bf16") for n in ("q", "k", "v")}
    del x
    t1 = time.perf_counter()
    oracle.attention_forward(f["q"], f["k"], f["v"], causal=lw.causal, scale=lw.scale)
    dl = time.perf_counter() - t1
    fl = nominal_fwd_flops(1, 1, lw.Sq, lw.Sk, lw.d, lw.causal)
    extra["long_causal_d128_fwd"] = {"value": round(fl / dl / 1e12, 5), "unit": "TFLOP/s", "seconds": round(dl, 2),
                                     "sample": "1 of 64 (batch, head) pairs, attention_forward"}
    del f
    # grouped-query decode: the whole workload
    dw = synth.get_workload("gqa_decode")
    x = synth.make_inputs(dw)
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v")}
    del x
    t2 = time.perf_counter()
    oracle.attention_forward(f["q"], f["k"], f["v"], causal=dw.causal, scale=dw.scale)
    dd = time.perf_counter() - t2
    alg = 2 * dw.B * dw.Hkv * dw.Sk * dw.d * 2 + 2 * dw.B * dw.Hq * dw.Sq * dw.d * 2 + dw.B * dw.Hq * dw.Sq * 4
    extra["gqa_decode_fwd"] = {"value": round(alg / dd / 1e9, 3), "unit": "GB/s", "seconds": round(dd, 2),
                               "sample": "the whole workload (bf16-equivalent bytes), attention_forward"}
    del f
    cores = host["blas_threads"] or host["affinity"] or os.cpu_count() or 1
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{heads} of {w.Hq} heads of {w.name} (S={w.Sq}, d={w.d}, causal), "
                      "attention_forward + attention_backward in float64 NumPy",
            "host": host, "other_workloads": extra}


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> None:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def mfma_ceiling(reps: int = 5) -> dict:
    """Sustained bf16 MFMA rate of the whole chip on a loop of independent
    32x32x16 MFMAs and nothing else (libcalib.so; one workgroup of four
    wavefronts per CU, about 3 ms per launch), median of `reps` launches after
    one warm-up, on changing random operands and on constant ones. The
    published dense peak assumes the top clock, which the chip does not hold
    under a full matrix load, least of all on changing data; these figures are
    what the kernels' MFMA fractions can be read against. Reported next to the
    published peak, never in place of it."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_38_amd", "libcalib.so"))
    lib.calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.calib_mfma_bf16.restype = ctypes.c_int
    blocks, nit = 256, 16384
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flop = blocks * 4 * nit * 8 * (2 * 32 * 32 * 16)
    res = {}
    for name, rnd in (("random_operands", 1), ("constant_operands", 0)):
        times = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = lib.calib_mfma_bf16(out.data_ptr(), blocks, nit, rnd, stream.cuda_stream)
            e1.record(stream)
            stream.synchronize()
            if st != 0:
                raise RuntimeError(f"calib_mfma_bf16 failed with status {st}")
            if r:
                times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        tf = flop / ms / 1e9
        res[name] = {"tflops": round(tf, 1), "frac_of_published_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "ms": round(ms, 3)}
    res.update({"tflops": res["random_operands"]["tflops"],
                "kernel": "mfma_loop_kernel: 8 independent 32x32x16 bf16 MFMA chains per wavefront, "
                          "4 wavefronts per CU", "launches": reps})
    return res


def coissue(nit: int = 512) -> dict:
    """How one SIMD shares its matrix pipe and vector ALU between two
    wavefronts (libcalib.so calib_coissue, one workgroup of 8 wavefronts per
    CU, shader-clock cycles per wavefront, medians over the chip): the
    forward's matrix stream (one MFMA per KB of LDS operand reads) alone and
    beside a softmax-shaped vector stream on the same SIMD, and the vector
    stream alone with one and with two wavefronts per SIMD, and the matrix
    stream on both wavefronts of every SIMD (both reading LDS)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_38_amd", "libcalib.so"))
    lib.calib_coissue.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.calib_coissue.restype = ctypes.c_int
    blocks = 256
    cyc = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ideal = nit * 64 * 32                         # 64 MFMAs of 32 cycles per round
    scores = 96 * nit                             # per vector wavefront (lane)
    res = {}
    for mode in range(5):
        for warm in (True, False):
            st = lib.calib_coissue(cyc.data_ptr(), out.data_ptr(), blocks, max(1, nit // 8) if warm else nit, mode,
                                   stream.cuda_stream)
            stream.synchronize()
            if st != 0:
                raise RuntimeError(f"calib_coissue failed with status {st}")
        c = cyc.view(blocks, 8).cpu()
        mat = sorted(c[:, :4].flatten().tolist()) if mode <= 1 else sorted(c.flatten().tolist()) if mode == 4 else []
        vec = sorted(c[:, 4:].flatten().tolist() if mode in (1, 2) else c.flatten().tolist()) if 1 <= mode <= 3 else []
        r = {}
        if mat:                                   # mode 4: two matrix wavefronts share each pipe
            r["matrix_pipe_frac"] = round(ideal * (2 if mode == 4 else 1) / mat[len(mat) // 2], 4)
        if vec:
            r["vector_cycles_per_score"] = round(vec[len(vec) // 2] / scores, 2)
        res[("matrix_alone", "matrix_with_vector", "vector_one_wave_per_simd", "vector_two_waves_per_simd",
             "matrix_two_waves_per_simd")[mode]] = r
    res["note"] = ("matrix stream: per MFMA pair one ds_read_b128 K fragment and two ds_read_b64_tr_b16 V halves, "
                   "two pairs ahead; vector stream per score: fma, exp2, sum-tree add, half a bf16 pack, fma; "
                   "32 cycles per 32x32x16 bf16 MFMA at the published peak")
    return res


def _read_counter_csv(d: str):
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection*.csv"), recursive=True):
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_counters(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                       copy_write_dir: str, command: str) -> None:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel by the
    ratio a plain 1 GiB copy reads for the same counters, and store per-kernel
    HBM bytes per launch under profiles/."""
    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return acc

    def copy_factor(rows, counter, nbytes=1 << 30):
        vals = [v for k, vs in per_kernel(rows, counter).items() for v in vs
                if "copy" in k.lower() or "elementwise" in k.lower()]
        vals = [v for v in vals if v > 0.25 * nbytes / 1024]
        if not vals:
            return None, None
        med = sorted(vals)[len(vals) // 2]
        return nbytes / (med * 1024.0), med

    fetch = per_kernel(_read_counter_csv(fetch_dir), "FETCH_SIZE")
    write = per_kernel(_read_counter_csv(write_dir), "WRITE_SIZE")
    ff, fcopy = copy_factor(_read_counter_csv(copy_fetch_dir), "FETCH_SIZE")
    wf, wcopy = copy_factor(_read_counter_csv(copy_write_dir), "WRITE_SIZE")
    for kern in KERNEL_SYMBOLS:
        fk = [v for k, vs in fetch.items() if kernel_matches(kern, k) for v in vs]
        wk = [v for k, vs in write.items() if kernel_matches(kern, k) for v in vs]
        if not fk or not wk or ff is None or wf is None:
            continue
        f_kib = sorted(fk)[len(fk) // 2]
        w_kib = sorted(wk)[len(wk) // 2]
        out = {"kernel": kern, "workload": workload, "source_sha": source_hash(kern),
               "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
               "copy_calibration": {"bytes": 1 << 30, "fetch_kib": fcopy, "write_kib": wcopy,
                                    "fetch_factor": ff, "write_factor": wf},
               "hbm_bytes_per_launch": int(f_kib * 1024 * ff + w_kib * 1024 * wf),
               "command": command}
        with open(counters_path(kern, workload), "w") as f:
            json.dump(out, f, indent=1)
        print(kern, out["hbm_bytes_per_launch"])


def summarize_pmc(workload: str, title: str, dirs, command: str, out_md: str = None) -> str:
    """Per-kernel shader counters from rocprofv3 --pmc runs (one directory per
    pass, each pass within the hardware's counter limits), averaged over the
    kernel's dispatches, with the figures derived from them:

    * clock: GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 / dispatch duration;
    * MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs; a
      32x32x16 bf16 MFMA counts 32 cycles) / (GRBM_GUI_ACTIVE / 8 * 1024), the
      MfmaUtil expression of rocprofiler's counter definitions;
    * VALU busy: SQ_ACTIVE_INST_VALU / 256 CUs / (GRBM_GUI_ACTIVE / 8), its
      VALUBusy expression;
    * executed MFMA work: SQ_INSTS_VALU_MFMA_MOPS_BF16 (or _F8) x 512 FLOP;
    * transcendental share: SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_VALU;
    * LDS bank conflicts: SQ_LDS_BANK_CONFLICT cycles per CU cycle;
    * with a second pass: the share of MFMA-busy cycles in which the vector
      ALU co-executes (SQ_VALU_MFMA_COEXEC_CYCLES), LDS activity and FIFO-full
      cycles per CU cycle, and the share of wave cycles spent waiting to issue
      an LDS instruction, waiting on anything, or issuing (per SQ_WAVE_CYCLES).

    Writes profiles/pmc__<workload>.md (or out_md) and returns its path."""
    per = {}         # short kernel name -> counter -> [values]
    durs = {}
    for d in dirs:
        for r in _read_counter_csv(d):
            k = _short_kernel_name(r.get("Kernel_Name", ""))
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            try:
                durs.setdefault(k, {})[(d, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            except (KeyError, ValueError):
                pass

    def mean(k, c):
        v = per.get(k, {}).get(c)
        return sum(v) / len(v) if v else None

    lines = [f"# rocprofv3 shader counters: {title}", "",
             "Commands (run from the repository root on one MI355X; one counter pass per run):", "", "```",
             command, "```", "",
             "Values are per dispatch, averaged over the dispatches of each kernel. Derived: clock = "
             "GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x "
             "1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE / 8 x 256 CUs); executed MFMA "
             "TFLOP = MOPS x 512; TRANS share = SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_VALU; LDS bank-conflict "
             "cycles per CU cycle = SQ_LDS_BANK_CONFLICT / (GRBM_GUI_ACTIVE / 8 x 256).", ""]
    names = sorted(per, key=lambda k: -(sum(durs.get(k, {}).values()) / max(1, len(durs.get(k, {})))))
    for k in names:
        c = per[k]
        dv = list(durs.get(k, {}).values())
        dur_us = sum(dv) / len(dv) / 1e3 if dv else None
        lines += [f"## {k}", "", "| counter | mean per dispatch |", "|---|---|"]
        for n in sorted(c):
            lines.append(f"| {n} | {mean(k, n):.6g} |")
        lines += ["", "| derived | value |", "|---|---|"]
        if dur_us:
            lines.append(f"| dispatch duration (us) | {dur_us:.1f} |")
        gui = mean(k, "GRBM_GUI_ACTIVE")
        if gui and dur_us:
            lines.append(f"| clock (GHz) | {gui / N_XCD / (dur_us * 1e3):.3f} |")
        if gui and mean(k, "SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            lines.append(f"| MFMA busy (%) | {100 * mean(k, 'SQ_VALU_MFMA_BUSY_CYCLES') / (gui / N_XCD * N_SIMD):.1f} |")
        if gui and mean(k, "SQ_ACTIVE_INST_VALU") is not None:
            lines.append(f"| VALU busy (%) | {100 * mean(k, 'SQ_ACTIVE_INST_VALU') / (gui / N_XCD * N_SIMD / 4):.1f} |")
        for mops, label in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", "bf16"), ("SQ_INSTS_VALU_MFMA_MOPS_F8", "fp8")):
            m = mean(k, mops)
            if m:
                lines.append(f"| executed MFMA work, {label} (TFLOP) | {m * 512 / 1e12:.4f} |")
                if dur_us:
                    lines.append(f"| executed MFMA rate, {label} (TFLOP/s) | {m * 512 / (dur_us * 1e-6) / 1e12:.1f} |")
        t, v = mean(k, "SQ_INSTS_VALU_TRANS_F32"), mean(k, "SQ_INSTS_VALU")
        if t is not None and v:
            lines.append(f"| TRANS share of VALU instructions (%) | {100 * t / v:.1f} |")
        b = mean(k, "SQ_LDS_BANK_CONFLICT")
        if b is not None and gui:
            lines.append(f"| LDS bank-conflict cycles per CU cycle | {b / (gui / N_XCD * N_SIMD / 4):.4f} |")
        co, mb = mean(k, "SQ_VALU_MFMA_COEXEC_CYCLES"), mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        if co is not None and mb:
            lines.append(f"| VALU co-executing with MFMA (% of MFMA-busy cycles) | {100 * co / mb:.1f} |")
        cu_cycles = gui / N_XCD * N_SIMD / 4 if gui else None
        for ctr, label in (("SQ_LDS_IDX_ACTIVE", "LDS active"), ("SQ_LDS_DATA_FIFO_FULL", "LDS data FIFO full"),
                           ("SQ_LDS_CMD_FIFO_FULL", "LDS command FIFO full")):
            x = mean(k, ctr)
            if x is not None and cu_cycles:
                lines.append(f"| {label} (% of CU cycles) | {100 * x / cu_cycles:.1f} |")
        wc = mean(k, "SQ_WAVE_CYCLES")
        for ctr, label in (("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction"),
                           ("SQ_WAIT_ANY", "waiting on anything"), ("SQ_ACTIVE_INST_ANY", "issuing")):
            x = mean(k, ctr)
            if x is not None and wc:
                lines.append(f"| wave cycles {label} (%) | {100 * x / wc:.1f} |")
        lines.append("")
    out_md = out_md or os.path.join(PROFILES, f"pmc__{workload}.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")
    return out_md


def _demangle(name: str) -> str:
    if not name.startswith("_Z"):
        return name
    import shutil
    import subprocess
    tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    if tool is None:
        return name
    r = subprocess.run([tool, name], capture_output=True, text=True)
    out = r.stdout.strip()
    if out and out != name:
        return out
    # older demanglers do not know the bf16 type code: take the kernel's own
    # identifier, the last <length><name> of the nested name
    import re
    m = re.match(r"_ZN(?:\d+[A-Za-z_]\w*?)*?(\d+)([A-Za-z_]\w*?)E", name)
    if m is None:
        return name
    pos, last = 3, name
    while pos < len(name) and name[pos].isdigit():
        n = re.match(r"\d+", name[pos:]).group(0)
        last = name[pos + len(n):pos + len(n) + int(n)]
        pos += len(n) + int(n)
    return last


def _short_kernel_name(name: str) -> str:
    # "void attn::(anonymous namespace)::bwd_dq_kernel<128, true>(attn::...)" -> "bwd_dq_kernel<128, true>"
    name = _demangle(name).replace("void ", "").replace("attn::(anonymous namespace)::", "")
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].strip()


def summarize_stats(stats_csv: str, title: str, out_md: str, command: str) -> None:
    """Markdown table of a rocprofv3 --stats kernel_stats.csv, written to out_md."""
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel statistics: {title}", "",
             "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short_kernel_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "step", "step_fused", "fwd", "decode", "varlen", "fp8", "fp8_decode", "f32",
                                       "d64", "gqa_prefill", "mfma_ceiling", "coissue"], default="all")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ARG",
                    help="WORKLOAD TITLE DIR [DIR ...]")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=5,
                    metavar=("WORKLOAD", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "TITLE", "OUT_MD"))
    ap.add_argument("--command", default="")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, command=args.command)
        return 0
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats, command=args.command)
        return 0
    if args.summarize_pmc:
        if len(args.summarize_pmc) < 3:
            ap.error("--summarize-pmc needs WORKLOAD TITLE DIR [DIR ...]")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summarize_pmc[2:], command=args.command)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0

    import torch
    import exact_io_aware_38_amd as attn
    attn.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    result = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic"}
    if args.only in ("all", "step"):
        w, ms, total, kern, dom, sp = bench_step(attn, args.steps, args.warmup)
        print(f"# step: {ms:.3f} ms, kernels {kern}", file=sys.stderr, flush=True)
        result.update({"value": round(total / ms / 1e9, 2), "ms_per_step": round(ms, 4), "spread": sp,
                       "frac_of_peak": round(total / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                       "config": {"workload": w.name, "B": w.B, "H": w.Hq, "S": w.Sq, "d": w.d,
                                  "causal": w.causal, "step": "attn_fwd + attn_bwd",
                                  "nominal_tflop_per_step": round(total / 1e12, 4)},
                       "roofline": roofline(dom, w, kern[dom]),
                       "kernels_ms": {k: round(v, 4) for k, v in kern.items()}})
        torch.cuda.empty_cache()
    if args.only in ("all", "step_fused"):
        # the single-pass backward with atomically summed dQ on the same step, for comparison
        w2, ms2, total2, kern2, dom2, sp2 = bench_step(attn, max(3, args.steps // 4), 2, fused=True)
        result["step_fused"] = {
            "step": "attn_fwd + attn_bwd_fused", "ms": round(ms2, 4), "spread": sp2,
            "tflops": round(total2 / ms2 / 1e9, 2), "frac_of_peak": round(total2 / ms2 / 1e9 / PEAK_BF16_TFLOPS, 4),
            "roofline": roofline(dom2, w2, kern2[dom2]), "kernels_ms": {k: round(v, 4) for k, v in kern2.items()}}
        print(f"# step, fused backward: {ms2:.3f} ms, kernels {kern2}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "fwd"):
        result["fwd"] = bench_fwd(attn, args.steps, args.warmup)
        print(f"# fwd: {result['fwd']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "f32"):
        result["single_head_f32"] = bench_fwd(attn, max(args.steps, 20), args.warmup, "single_head_f32")
        print(f"# single-head fp32: {result['single_head_f32']['ms']} ms", file=sys.stderr, flush=True)
    if args.only in ("all", "d64"):
        result["multihead_d64"] = bench_multihead_d64(attn, args.steps, args.warmup)
        print("# multi-head d64: " + ", ".join(f"{k} {result['multihead_d64'][k]['ms']} ms" for k in C2_VARIANTS),
              file=sys.stderr, flush=True)
    if args.only in ("all", "gqa_prefill"):
        result["gqa_prefill"] = bench_fwd(attn, args.steps, args.warmup, "gqa_prefill")
        print(f"# gqa prefill: {result['gqa_prefill']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "fp8"):
        result["fp8"] = bench_fp8(attn, args.steps, args.warmup)
        print(f"# fp8: {result['fp8']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "fp8_decode"):
        result["fp8_decode"] = bench_fp8_decode(attn, max(args.steps, 20), args.warmup)
        print(f"# fp8 decode: {result['fp8_decode']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        result["decode"] = bench_decode(attn, max(args.steps, 20), args.warmup)
        print(f"# decode: {result['decode']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "varlen"):
        result["varlen"] = bench_varlen(attn, args.steps, args.warmup)
        print(f"# varlen: {result['varlen']['ms']} ms", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if args.only in ("all", "mfma_ceiling"):
        result["mfma_ceiling"] = mfma_ceiling()
        print(f"# sustained MFMA loop: {result['mfma_ceiling']['tflops']} TFLOP/s", file=sys.stderr, flush=True)
        # the bf16 MFMA-bound rooflines of this run read against the sustained rate as well
        ceil = result["mfma_ceiling"]["tflops"]
        against = {}
        for key, sub in (("step", result), ("fwd", result.get("fwd")), ("gqa_prefill", result.get("gqa_prefill")),
                         ("varlen", result.get("varlen"))):
            rl = (sub or {}).get("roofline")
            if rl and rl.get("bound") == "mfma" and rl.get("peak") == PEAK_BF16_TFLOPS and ceil:
                against[f"{key}:{rl['kernel']}"] = round(rl["achieved"] / ceil, 4)
        result["mfma_ceiling"]["dominant_kernels_over_sustained"] = against
    if args.only == "coissue":
        result["coissue"] = coissue()
        r = result["coissue"]
        result.update({"value": r["matrix_with_vector"]["matrix_pipe_frac"], "unit": "fraction", "ms_per_step": None,
                       "config": {"workload": "coissue"}})
    if args.only == "mfma_ceiling":
        r = result["mfma_ceiling"]
        result.update({"value": r["tflops"], "ms_per_step": r["random_operands"]["ms"],
                       "config": {"workload": "mfma_loop"}})
    if args.only == "varlen":
        result.update({"value": result["varlen"]["tflops"], "ms_per_step": result["varlen"]["ms"],
                       "config": {"workload": result["varlen"]["workload"]},
                       "roofline": result["varlen"]["roofline"]})
    if args.only == "fp8_decode":
        result.update({"value": result["fp8_decode"]["gbs"], "unit": "GB/s", "dtype": "e4m3",
                       "ms_per_step": result["fp8_decode"]["ms"],
                       "config": {"workload": result["fp8_decode"]["workload"]},
                       "roofline": result["fp8_decode"]["roofline"]})
    if args.only == "fp8":
        result.update({"value": result["fp8"]["tflops"], "ms_per_step": result["fp8"]["ms"], "dtype": "e4m3",
                       "config": {"workload": result["fp8"]["workload"]}, "roofline": result["fp8"]["roofline"]})
    for key, sub in (("fwd", "fwd"), ("f32", "single_head_f32"), ("gqa_prefill", "gqa_prefill")):
        if args.only == key:
            r = result[sub]
            result.update({"value": r["tflops"], "ms_per_step": r["ms"], "spread": r["spread"],
                           "dtype": r["dtype"], "config": {"workload": r["workload"]}, "roofline": r["roofline"]})
    if args.only == "d64":
        r = result["multihead_d64"]["causal"]
        result.update({"value": r["tflops"], "ms_per_step": r["ms"], "spread": r["spread"],
                       "config": {"workload": r["workload"]}, "roofline": r["roofline"]})
    if args.only == "decode":
        result.update({"value": result["decode"]["gbs"], "unit": "GB/s", "ms_per_step": result["decode"]["ms"],
                       "config": {"workload": result["decode"]["workload"]},
                       "roofline": result["decode"]["roofline"]})
    if not args.no_cpu_baseline and args.only in ("all", "step"):
        import synth
        print("# cpu baseline (oracle on sampled heads) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(synth.get_workload("train_causal_d128"))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
