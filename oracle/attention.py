"""Plain, slow, obviously correct FP64 attention -- test infrastructure only.

Nothing in the library imports this module; only tests, the smoke check and
the benchmark's CPU-baseline leg do. Every function upcasts its inputs to
float64 and follows a definition or a recurrence stated on the source pages:

* [P1] "Flash Attention FA1->FA4 / pre-training practice" (wmrh.cn/news/479911)
* [P2] "AI 大模型之 FlashAttention_01" (security.zone.ci/secarticles/wx/581217.html)

Notation follows the pages: scores s = scale * q.k, running max m, running
denominator l, unnormalised output accumulator u, output O = u / l, and the
per-row logsumexp (natural log) that the forward keeps for the backward.

Readings taken where the pages leave a step open (all listed in the design
notes):

* causal = 1 is the top-left triangle (key j visible to query i iff j <= i);
  causal = 2 is bottom-right alignment (j <= i + Sk - Sq), the form of the
  masked gradient example of [P2] "训练与部署 注意力反向的完整链式关系",
  where the first of two queries may not read the third of three keys.
* A row with no visible key has no softmax. [P2] "瓦片状态如何保持精确语义"
  asks for an explicit rule; strict mode raises (the teaching check of [P2]
  "工程实操" rejects such rows), the default defined mode returns O = 0,
  lse = -inf and zero gradients.
* GQA groups are contiguous: query head h reads KV head h // (Hq // Hkv).

Every function here is pinned by tests against values printed on the pages,
closed forms, library routines and central differences, not against itself.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "FullyMaskedRowError", "visible_mask", "attention_forward",
    "attention_backward", "online_softmax_forward", "merge_states",
    "attention_forward_varlen", "attention_backward_varlen", "philox4x32_10",
    "dropout_threshold", "dropout_keep_mask",
]


class FullyMaskedRowError(ValueError):
    """Raised in strict mode when a query row can see no key at all."""


def _scale(scale: Optional[float], d: int) -> float:
    # [P1] §1.1: scores are divided by sqrt(d_k) unless a scale is given.
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def visible_mask(Sq: int, Sk: int, causal: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Boolean [n_rows, Sk]: True where query row i may attend key j.

    causal 0: every key; 1: j <= i; 2: j <= i + Sk - Sq. ``rows`` selects
    absolute query indices (default: all Sq rows).
    """
    i = np.arange(Sq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Sk, dtype=np.int64)
    if causal == 0:
        return np.ones((i.size, Sk), dtype=bool)
    if causal == 1:
        return j[None, :] <= i[:, None]
    if causal == 2:
        return j[None, :] <= (i[:, None] + (Sk - Sq))
    raise ValueError(f"causal must be 0, 1 or 2, got {causal}")


def _group(Hq: int, Hkv: int) -> int:
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    return Hq // Hkv


_PHILOX_MUL = (0xD2511F53, 0xCD9E8D57)
_PHILOX_WEYL = (0x9E3779B9, 0xBB67AE85)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), vectorised over the leading axes.

    counter: integers [..., 4] below 2^32; key: (k0, k1). Each round forms the
    64-bit products of the first and third counter words with the two round
    multipliers; the new words are (high of the second product xor word 1 xor
    k0, low of the second product, high of the first product xor word 3 xor k1,
    low of the first product). The key advances by the two Weyl constants after
    every round. Returns uint64 [..., 4] holding 32-bit words.
    """
    c = [np.asarray(counter, dtype=np.uint64)[..., w] & _U32 for w in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = c[0] * np.uint64(_PHILOX_MUL[0])          # < 2^64: exact in uint64
        p1 = c[2] * np.uint64(_PHILOX_MUL[1])
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & _U32,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & _U32]
        k0 = (k0 + _PHILOX_WEYL[0]) & 0xFFFFFFFF
        k1 = (k1 + _PHILOX_WEYL[1]) & 0xFFFFFFFF
    return np.stack(c, axis=-1)


def dropout_threshold(p: float) -> int:
    """The byte threshold of a dropout probability: round(256 p) with p taken
    in single precision (the library's argument type), ties to even."""
    p32 = np.float32(p)
    if not np.isfinite(p32) or p32 < 0 or p32 >= 1:
        raise ValueError(f"dropout probability {p} not in [0, 1)")
    thr = int(np.rint(p32 * np.float32(256.0)))
    if thr > 255:
        raise ValueError(f"dropout probability {p} rounds to 256/256")
    return thr


def dropout_keep_mask(B: int, Hq: int, Sq: int, Sk: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep mask [B, Hq, Sq, Sk] of the dropout contract.

    [P2] "接口与实现约束" asks that, with dropout on, the mapping to random
    numbers be part of the contract between the forward and the backward;
    the pages name no generator. Reading taken: Philox4x32-10 keyed by the
    64-bit seed (low word first); the 4x4 block of query rows 4a..4a+3 and
    keys 4c..4c+3 of query head h in batch b takes counter (c, a, b Hq + h,
    offset); byte t of output word w decides query 4a+w, key 4c+t, which is
    kept when the byte is at least round(256 p).
    """
    thr = dropout_threshold(p)
    na, nc = (Sq + 3) // 4, (Sk + 3) // 4
    bh, a, c = np.meshgrid(np.arange(B * Hq), np.arange(na), np.arange(nc), indexing="ij")
    ctr = np.stack([c, a, bh, np.full_like(c, offset)], axis=-1)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))   # [BH, na, nc, 4]
    shifts = np.arange(4, dtype=np.uint64) * np.uint64(8)
    byte = (words[..., :, None] >> shifts) & np.uint64(0xFF)                     # [BH, na, nc, w, t]
    full = byte.transpose(0, 1, 3, 2, 4).reshape(B * Hq, 4 * na, 4 * nc)         # rows 4a+w, cols 4c+t
    return (full[:, :Sq, :Sk] >= thr).reshape(B, Hq, Sq, Sk)


def _dropout_factor(dropout, B, Hq, Sq, Sk):
    """Z = keep / (1 - thr/256) as float64 [B, Hq, Sq, Sk], or None."""
    if dropout is None:
        return None
    p, seed, offset = dropout
    thr = dropout_threshold(p)
    keep = dropout_keep_mask(B, Hq, Sq, Sk, p, seed, offset)
    return keep.astype(np.float64) / (1.0 - thr / 256.0)


def attention_forward(q, k, v, *, causal: int = 0, scale: Optional[float] = None,
                      strict: bool = False, rows: Optional[Sequence[int]] = None,
                      Sq: Optional[int] = None, dropout=None) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * Q K^T, masked) V by its definition, in float64.

    q: [B, Hq, n, d]; k: [B, Hkv, Sk, d]; v: [B, Hkv, Sk, dv]. When ``rows`` is
    given, q holds just those absolute query rows of a problem with ``Sq``
    rows (the mask depends on the absolute index). Returns (O [B, Hq, n, dv],
    lse [B, Hq, n]) with lse the natural-log logsumexp of the visible scores.

    Definition: [P1] §1.1 (Attention = softmax(QK^T/sqrt(d_k)) V); the mask is
    applied before the row maximum as [P2] "瓦片状态如何保持精确语义" requires;
    the max is subtracted before exponentiation, which leaves the softmax
    unchanged and keeps exp finite for the large scores of [P2] "工程实操".

    ``dropout=(p, seed, offset)`` multiplies the probabilities by
    Z = keep / (1 - thr/256) (``dropout_keep_mask``) before V; lse stays the
    logsumexp of the undropped scores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, n, d = q.shape
    _, Hkv, Sk, _ = k.shape
    g = _group(Hq, Hkv)
    c = _scale(scale, d)
    if rows is None:
        Sq_ = n if Sq is None else Sq
        vis = visible_mask(Sq_, Sk, causal)
    else:
        if Sq is None:
            raise ValueError("Sq is required with rows")
        vis = visible_mask(Sq, Sk, causal, rows)
    if vis.shape[0] != n:
        raise ValueError("rows and q disagree in length")
    dv = v.shape[-1]
    o = np.zeros((B, Hq, n, dv))
    lse = np.full((B, Hq, n), -np.inf)
    empty = ~vis.any(axis=1)
    if strict and empty.any():
        raise FullyMaskedRowError(f"{int(empty.sum())} query row(s) see no key")
    if dropout is not None and rows is not None:
        raise ValueError("dropout applies to whole problems, not row subsets")
    Z = _dropout_factor(dropout, B, Hq, n, Sk)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            s = c * (q[b, h] @ k[b, hk].T)              # [n, Sk]
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)          # row max over visible keys
            ok = np.isfinite(m)
            e = np.zeros_like(s)
            e[ok] = np.exp(s[ok] - m[ok, None])         # masked entries give exp(-inf) = 0
            l = e.sum(axis=1)
            p = np.zeros_like(s)
            p[ok] = e[ok] / l[ok, None]
            if Z is not None:
                p = p * Z[b, h]
            o[b, h] = p @ v[b, hk]
            lse[b, h, ok] = m[ok] + np.log(l[ok])
    return o, lse


def attention_backward(q, k, v, do, *, causal: int = 0, scale: Optional[float] = None,
                       return_intermediates: bool = False, dropout=None) -> Dict[str, np.ndarray]:
    """Analytic gradients of O = softmax(scale Q K^T, masked) V, in float64.

    Follows the chain of [P2] "反向传播为什么可以重算" and "训练与部署":
    dV = P^T dO, dP = dO V^T, dS from the softmax Jacobian
    (dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)), then dQ = scale dS K and
    dK = scale dS^T Q. P is rebuilt from the definition here. Grouped heads
    sum their dK/dV into the shared KV head.

    Returns dq [B,Hq,Sq,d], dk [B,Hkv,Sk,d], dv [B,Hkv,Sk,dv]; with
    ``return_intermediates`` also p, ds (per query head, [B,Hq,Sq,Sk]) and
    D (the Jacobian row term sum_k P_ik dP_ik, [B,Hq,Sq]).

    With ``dropout=(p, seed, offset)`` the output is (P o Z) V, so by the chain
    rule dV = (P o Z)^T dO, the gradient reaching P is Z o (dO V^T), and the
    softmax Jacobian acts on that (D is then sum_k P_ik Z_ik (dO V^T)_ik).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    g = _group(Hq, Hkv)
    c = _scale(scale, d)
    vis = visible_mask(Sq, Sk, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    Z = _dropout_factor(dropout, B, Hq, Sq, Sk)
    extra = {}
    if return_intermediates:
        extra = {"p": np.zeros((B, Hq, Sq, Sk)), "ds": np.zeros((B, Hq, Sq, Sk)),
                 "D": np.zeros((B, Hq, Sq))}
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            s = c * (q[b, h] @ k[b, hk].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            ok = np.isfinite(m)
            p = np.zeros_like(s)
            p[ok] = np.exp(s[ok] - m[ok, None])
            p[ok] /= p[ok].sum(axis=1, keepdims=True)
            pz = p if Z is None else p * Z[b, h]
            dv[b, hk] += pz.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            if Z is not None:
                dp = dp * Z[b, h]
            D = (p * dp).sum(axis=1)                    # Jacobian row term
            ds = p * (dp - D[:, None])                  # zero wherever p is zero (masked)
            dq[b, h] = c * (ds @ k[b, hk])
            dk[b, hk] += c * (ds.T @ q[b, h])
            if return_intermediates:
                extra["p"][b, h] = p
                extra["ds"][b, h] = ds
                extra["D"][b, h] = D
    out = {"dq": dq, "dk": dk, "dv": dv}
    out.update(extra)
    return out


def online_softmax_forward(q, k, v, *, tile: int, causal: int = 0,
                           scale: Optional[float] = None, trace: bool = False):
    """The tiled online-softmax recurrence in float64, key tile by key tile.

    For every query row it keeps the running max m (init -inf), the running
    denominator l (init 0) and the unnormalised accumulator u (init 0). For a
    new key tile with scores s it sets m_new = max(m, max s), rescales the old
    l and u by exp(m - m_new), adds exp(s - m_new) and exp(s - m_new) @ V, and
    at the end returns O = u / l and lse = m + ln l. This is the update of [P1]
    §1.2 in the unnormalised form of [P2] §4.1 and "瓦片状态如何保持精确语义",
    extended from one query to all rows, masks and any tile length (the last
    tile may be short). Masked scores are -inf before the max. A row whose
    running max is still -inf contributes nothing (its factor exp(m - m_new) is
    taken as 1 and its weights as 0), and ends with O = 0, lse = -inf.

    With ``trace`` it also returns, per tile, the (m, l, u) state of every row
    of the first (batch, head).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if tile < 1:
        raise ValueError("tile must be >= 1")
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    g = _group(Hq, Hkv)
    c = _scale(scale, d)
    vis = visible_mask(Sq, Sk, causal)
    dv = v.shape[-1]
    o = np.zeros((B, Hq, Sq, dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    states: List[Tuple[np.ndarray, np.ndarray, np.ndarray]] = []
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            m = np.full(Sq, -np.inf)
            l = np.zeros(Sq)
            u = np.zeros((Sq, dv))
            for start in range(0, Sk, tile):
                stop = min(start + tile, Sk)
                s = c * (q[b, h] @ k[b, hk, start:stop].T)
                s = np.where(vis[:, start:stop], s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                a = np.ones(Sq)
                a[live] = np.exp(m[live] - m_new[live])     # exp(-inf) = 0 on a row's first live tile
                p = np.zeros_like(s)
                p[live] = np.exp(s[live] - m_new[live, None])
                u = a[:, None] * u + p @ v[b, hk, start:stop]
                l = a * l + p.sum(axis=1)
                m = m_new
                if trace and b == 0 and h == 0:
                    states.append((m.copy(), l.copy(), u.copy()))
            ok = l > 0
            o[b, h, ok] = u[ok] / l[ok, None]
            lse[b, h, ok] = m[ok] + np.log(l[ok])
    if trace:
        return o, lse, states
    return o, lse


def merge_states(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two normalised partial results over disjoint key sets.

    The update of [P1] §1.2 written for a whole block at once: with
    M = max(lse_a, lse_b), the merged weight of each part is exp(lse_x - M),
    lse = M + ln(sum of weights) and O is the weight-averaged O. Parts with
    lse = -inf (no visible key) weigh 0; if both are empty the result is
    O = 0, lse = -inf.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(lse_a, lse_b)
    live = np.isfinite(M)
    wa = np.zeros_like(M)
    wb = np.zeros_like(M)
    wa[live] = np.exp(lse_a[live] - M[live])
    wb[live] = np.exp(lse_b[live] - M[live])
    tot = wa + wb
    o = np.zeros(np.broadcast_shapes(o_a.shape, o_b.shape))
    lse = np.full(M.shape, -np.inf)
    o[live] = (wa[live, None] * o_a[live] + wb[live, None] * o_b[live]) / tot[live, None]
    lse[live] = M[live] + np.log(tot[live])
    return o, lse


def _offsets(cu, name: str) -> List[int]:
    cu = [int(x) for x in cu]
    if len(cu) < 2 or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError(f"{name} must start at 0 and never decrease, got {cu}")
    return cu


def attention_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: int = 0,
                             scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over a packed batch of sequences of different lengths.

    q: [Hq, total_q, d]; k, v: [Hkv, total_k, d(v)], sequences back to back:
    sequence b owns packed query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
    and packed key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.

    [P2] "接口与实现约束" asks a ragged layout to keep the logical row number
    apart from the packed one. Reading taken: every sequence is its own
    attention problem (no row sees a key of another sequence), and the causal
    masks compare logical positions, i.e. the packed row minus the sequence's
    first packed row. Each sequence is cut out and handed to
    ``attention_forward``. A sequence without keys gets O = 0 and lse = -inf
    (the defined mode for rows that see nothing). Returns (O [Hq, total_q,
    dv], lse [Hq, total_q]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = _offsets(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _offsets(cu_seqlens_k, "cu_seqlens_k")
    if len(cu_q) != len(cu_k) or cu_q[-1] != q.shape[1] or cu_k[-1] != k.shape[1]:
        raise ValueError("offsets disagree with the packed tensors")
    Hq, total_q, _ = q.shape
    o = np.zeros((Hq, total_q, v.shape[-1]))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        qs = slice(cu_q[b], cu_q[b + 1])
        ks = slice(cu_k[b], cu_k[b + 1])
        ob, lb = attention_forward(q[None, :, qs], k[None, :, ks], v[None, :, ks],
                                   causal=causal, scale=scale)
        o[:, qs] = ob[0]
        lse[:, qs] = lb[0]
    return o, lse


def attention_backward_varlen(q, k, v, do, cu_seqlens_q, cu_seqlens_k, *, causal: int = 0,
                              scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gradients of ``attention_forward_varlen``, sequence by sequence.

    Same layout and reading as the forward: each sequence's dq, dk, dv come
    from ``attention_backward`` on that sequence alone, and since no row sees
    another sequence's keys, nothing crosses sequence boundaries. Key rows of
    a sequence without queries get zero dk and dv.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cu_q = _offsets(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _offsets(cu_seqlens_k, "cu_seqlens_k")
    if len(cu_q) != len(cu_k) or cu_q[-1] != q.shape[1] or cu_k[-1] != k.shape[1]:
        raise ValueError("offsets disagree with the packed tensors")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu_q) - 1):
        qs = slice(cu_q[b], cu_q[b + 1])
        ks = slice(cu_k[b], cu_k[b + 1])
        g = attention_backward(q[None, :, qs], k[None, :, ks], v[None, :, ks], do[None, :, qs],
                               causal=causal, scale=scale)
        dq[:, qs] = g["dq"][0]
        dk[:, ks] = g["dk"][0]
        dv[:, ks] = g["dv"][0]
    return {"dq": dq, "dk": dk, "dv": dv}
