"""Seeded synthetic inputs for exact attention.

This module is shared by the FP64 oracle tests, the GPU parity tests and the
benchmark. It only draws random numbers and rounds them to the storage dtype;
it holds none of the attention arithmetic, so neither side of a parity check
can lean on the other through it.

Recipe (the same for every consumer):

* generator ``numpy.random.Generator(PCG64(seed))``;
* draw order: q, k, v, then dO (only when a backward is wanted), then the
  outlier row indices;
* each tensor is drawn as i.i.d. N(0, 1) with ``standard_normal(dtype=float32)``;
* outlier rows (the long-context workload): per (batch, head), a fraction of
  the query rows chosen without replacement is multiplied by a factor in fp32,
  before the cast to the storage dtype, which pushes scores past ln(FLT_MAX);
* bf16 storage is round-to-nearest-even of the fp32 draw, kept as raw uint16
  bit patterns. Consumers upcast those exact values.

Packed variable-length batches (``VarlenWorkload``): the sequence lengths are
drawn first, as integers uniform in [min_len, max_len] (query and key lengths
equal unless the workload lists them), then q, k, v, dO as above but in the
packed head-major shapes [H, total, d].
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "make_inputs", "to_f64", "get_workload", "VarlenWorkload", "VARLEN_WORKLOADS",
    "varlen_lengths", "make_varlen_inputs", "cu_seqlens",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bf16 bit patterns as uint16. NaN inputs are not expected
    (the generator never draws them) and are not given special treatment.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return f32_from_bf16_bits(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclass(frozen=True)
class Workload:
    """Shape, dtype, mask and seed of one synthetic attention problem.

    Tensors are row-major ``[B, H, S, d]``: q/o/dO are ``[B, Hq, Sq, d]``,
    k/v are ``[B, Hkv, Sk, d]``.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: str            # "f32" or "bf16"
    causal: int           # 0 none, 1 top-left (j <= i), 2 bottom-right (j <= i + Sk - Sq)
    seed: int
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    backward: bool = False
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads the library is specified and measured on.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("single_head_f32", 1, 1, 1, 256, 256, 64, "f32", 0, seed=1,
             note="single head, non-causal, fp32"),
    Workload("multihead_d64", 4, 16, 16, 2048, 2048, 64, "bf16", 0, seed=2,
             note="multi-head prefill d=64, non-causal"),
    Workload("multihead_d64_causal", 4, 16, 16, 2048, 2048, 64, "bf16", 1, seed=2,
             note="multi-head prefill d=64, causal"),
    Workload("multihead_d64_ragged", 4, 16, 16, 2048, 2000, 64, "bf16", 0, seed=2,
             note="multi-head prefill d=64, ragged K/V length 2000, non-causal"),
    Workload("multihead_d64_ragged_causal", 4, 16, 16, 2048, 2000, 64, "bf16", 1, seed=2,
             note="multi-head prefill d=64, ragged K/V length 2000, causal"),
    Workload("long_causal_d128", 2, 32, 32, 8192, 8192, 128, "bf16", 1, seed=3,
             outlier_frac=0.01, outlier_scale=30.0,
             note="long-context causal prefill, 1% of query rows x30"),
    Workload("gqa_prefill", 1, 32, 8, 4096, 4096, 128, "bf16", 1, seed=4,
             note="grouped-query prefill, 4 query heads per KV head"),
    Workload("gqa_decode", 16, 32, 8, 1, 32768, 128, "bf16", 0, seed=40,
             note="grouped-query decode, one query row against a 32768-key cache"),
    Workload("train_causal_d128", 1, 32, 32, 8192, 8192, 128, "bf16", 1, seed=5,
             backward=True, note="training forward + backward, causal"),
]}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, *, backward: Optional[bool] = None) -> Dict[str, np.ndarray]:
    """Draw q, k, v (and dO) for a workload.

    Returns storage arrays: float32 for "f32", uint16 bf16 bit patterns for
    "bf16". Also returns ``outlier_rows`` (int64 ``[B, Hq, n]``) when the
    workload scales outlier rows.
    """
    want_do = w.backward if backward is None else backward
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((w.B, w.Hq, w.Sq, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Sk, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Sk, w.d), dtype=np.float32)
    out = {}
    if want_do:
        out["do"] = _store(rng.standard_normal((w.B, w.Hq, w.Sq, w.d), dtype=np.float32), w.dtype)
    if w.outlier_frac > 0.0:
        n = int(round(w.outlier_frac * w.Sq))
        rows = np.empty((w.B, w.Hq, n), dtype=np.int64)
        for b in range(w.B):
            for h in range(w.Hq):
                rows[b, h] = np.sort(rng.choice(w.Sq, size=n, replace=False))
                q[b, h, rows[b, h], :] *= np.float32(w.outlier_scale)
        out["outlier_rows"] = rows
    out["q"] = _store(q, w.dtype)
    out["k"] = _store(k, w.dtype)
    out["v"] = _store(v, w.dtype)
    return out


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of sequences of different lengths.

    Either explicit ``lens_q``/``lens_k`` tuples, or ``B`` lengths drawn
    uniformly in [min_len, max_len] (the same for queries and keys).
    Tensors are packed head-major: q/o/dO ``[Hq, total_q, d]``, k/v
    ``[Hkv, total_k, d]``.
    """
    name: str
    Hq: int
    Hkv: int
    d: int
    dtype: str
    causal: int
    seed: int
    B: int = 0
    min_len: int = 0
    max_len: int = 0
    lens_q: Optional[tuple] = None
    lens_k: Optional[tuple] = None
    backward: bool = False
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


VARLEN_WORKLOADS: Dict[str, VarlenWorkload] = {w.name: w for w in [
    VarlenWorkload("varlen_mix_causal_d128", 32, 32, 128, "bf16", 1, seed=7, B=16, min_len=512,
                   max_len=3584, backward=True,
                   note="16 causal sequences of 512..3584 tokens (mean 2048) packed back to back"),
]}


def varlen_lengths(w: VarlenWorkload):
    """(lens_q, lens_k) of a packed workload, as lists of ints."""
    if w.lens_q is not None:
        lk = w.lens_q if w.lens_k is None else w.lens_k
        return list(w.lens_q), list(lk)
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = rng.integers(w.min_len, w.max_len + 1, size=w.B).tolist()
    return lens, list(lens)


def cu_seqlens(lens):
    """Offsets [0, l0, l0 + l1, ...] of packed sequences."""
    out = [0]
    for x in lens:
        out.append(out[-1] + int(x))
    return out


def make_varlen_inputs(w: VarlenWorkload, *, backward: Optional[bool] = None) -> Dict[str, np.ndarray]:
    """Packed q, k, v (and dO) plus ``cu_seqlens_q``/``cu_seqlens_k`` for a workload."""
    want_do = w.backward if backward is None else backward
    lq, lk = varlen_lengths(w)
    tq, tk = sum(lq), sum(lk)
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000003))
    q = rng.standard_normal((w.Hq, tq, w.d), dtype=np.float32)
    k = rng.standard_normal((w.Hkv, tk, w.d), dtype=np.float32)
    v = rng.standard_normal((w.Hkv, tk, w.d), dtype=np.float32)
    out = {"q": _store(q, w.dtype), "k": _store(k, w.dtype), "v": _store(v, w.dtype),
           "cu_seqlens_q": np.asarray(cu_seqlens(lq), dtype=np.int64),
           "cu_seqlens_k": np.asarray(cu_seqlens(lk), dtype=np.int64)}
    if want_do:
        out["do"] = _store(rng.standard_normal((w.Hq, tq, w.d), dtype=np.float32), w.dtype)
    return out
