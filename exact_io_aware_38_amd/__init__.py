"""Exact IO-aware attention for MI355X (gfx950): Python binding of libattn.so.

This module only marshals arguments: it passes device pointers of PyTorch
tensors and the current HIP stream to the C ABI declared in
``include/attn.h``. Every step of the computation runs in the library's HIP
kernels. If the library has not been built, every call raises; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "ATTN_F32", "ATTN_BF16", "AttnError", "lib", "library_path", "fwd", "bwd",
    "fwd_workspace_bytes", "bwd_workspace_bytes", "strerror", "last_dispatch",
    "timing_start", "timing_stop", "fwd_varlen", "bwd_varlen", "fwd_varlen_workspace_bytes",
    "bwd_varlen_workspace_bytes", "fwd_dropout", "bwd_dropout", "dropout_mask",
    "fp8_padded_keys", "mxfp8_quantize_rows", "mxfp8_quantize_vt", "fwd_fp8", "fwd_fp8_workspace_bytes",
    "fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "bwd_fused_workspace_bytes",
]

ATTN_F32 = 0
ATTN_BF16 = 1
NOALLOC_SCRATCH_BYTES = 16 << 20      # the library's static scratch per GPU (attn_fwd_noalloc)
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_SHAPE = [_I] * 7                      # B, Hq, Hkv, Sq, Sk, d, causal
_IP = ctypes.POINTER(ctypes.c_int)
_VSHAPE = [_IP, _IP] + [_I] * 5        # cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal


class AttnError(RuntimeError):
    """A negative status returned by the C ABI."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m exact_io_aware_38_amd.build` "
                "(the HIP library is required; there is no fallback)")
        L = ctypes.CDLL(_LIB_PATH)
        L.attn_fwd_workspace_bytes.argtypes = _SHAPE + [_I]
        L.attn_fwd_workspace_bytes.restype = _Z
        L.attn_bwd_workspace_bytes.argtypes = _SHAPE + [_I]
        L.attn_bwd_workspace_bytes.restype = _Z
        L.attn_fwd.argtypes = [_P, _P, _P, _P, _P] + _SHAPE + [_F, _I, _P, _Z, _P]
        L.attn_fwd.restype = _I
        L.attn_fwd_noalloc.argtypes = [_P, _P, _P, _P, _P] + _SHAPE + [_F, _I, _P]
        L.attn_fwd_noalloc.restype = _I
        L.attn_bwd.argtypes = [_P] * 9 + _SHAPE + [_F, _I, _P, _Z, _P]
        L.attn_bwd.restype = _I
        L.attn_bwd_fused.argtypes = [_P] * 9 + _SHAPE + [_F, _I, _P, _Z, _P]
        L.attn_bwd_fused.restype = _I
        L.attn_bwd_fused_workspace_bytes.argtypes = _SHAPE + [_I]
        L.attn_bwd_fused_workspace_bytes.restype = _Z
        L.attn_fwd_varlen_workspace_bytes.argtypes = _VSHAPE + [_I]
        L.attn_fwd_varlen_workspace_bytes.restype = _Z
        L.attn_bwd_varlen_workspace_bytes.argtypes = _VSHAPE + [_I]
        L.attn_bwd_varlen_workspace_bytes.restype = _Z
        L.attn_fwd_varlen.argtypes = [_P, _P, _P, _P, _P] + _VSHAPE + [_F, _I, _P, _Z, _P]
        L.attn_fwd_varlen.restype = _I
        L.attn_bwd_varlen.argtypes = [_P] * 9 + _VSHAPE + [_F, _I, _P, _Z, _P]
        L.attn_bwd_varlen.restype = _I
        _DROP = [_F, ctypes.c_ulonglong, ctypes.c_uint]     # dropout_p, seed, offset
        L.attn_fwd_dropout.argtypes = [_P] * 5 + _SHAPE + [_F] + _DROP + [_P]
        L.attn_fwd_dropout.restype = _I
        L.attn_bwd_dropout.argtypes = [_P] * 9 + _SHAPE + [_F] + _DROP + [_P, _Z, _P]
        L.attn_bwd_dropout.restype = _I
        L.attn_dropout_mask.argtypes = [_P, _I, _I, _I, _I] + _DROP + [_P]
        L.attn_dropout_mask.restype = _I
        L.attn_fp8_padded_keys.argtypes = [_I]
        L.attn_fp8_padded_keys.restype = _I
        L.attn_mxfp8_quantize_rows.argtypes = [_P, _P, _P, ctypes.c_longlong, _I, _P]
        L.attn_mxfp8_quantize_rows.restype = _I
        L.attn_mxfp8_quantize_vt.argtypes = [_P, _P, _P, _I, _I, _I, _P]
        L.attn_mxfp8_quantize_vt.restype = _I
        L.attn_fwd_fp8_workspace_bytes.argtypes = _SHAPE
        L.attn_fwd_fp8_workspace_bytes.restype = _Z
        L.attn_fwd_fp8.argtypes = [_P] * 8 + _SHAPE + [_F, _P, _Z, _P]
        L.attn_fwd_fp8.restype = _I
        L.attn_strerror.argtypes = [_I]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_last_dispatch.argtypes = [ctypes.c_char_p, _Z]
        L.attn_last_dispatch.restype = _I
        L.attn_timing_start.argtypes = []
        L.attn_timing_start.restype = _I
        L.attn_timing_stop.argtypes = [ctypes.c_char_p, _Z]
        L.attn_timing_stop.restype = _I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def last_dispatch() -> str:
    """What the calling thread's last successful call launched."""
    n = lib().attn_last_dispatch(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    lib().attn_last_dispatch(buf, n + 1)
    return buf.value.decode()


def timing_start() -> None:
    """Start recording per-kernel device time for this thread's calls."""
    lib().attn_timing_start()


def timing_stop() -> dict:
    """Stop recording; returns {kernel: (launches, total_ms)} (waits for the events)."""
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib().attn_timing_stop(buf, len(buf))
    if n < 0:
        raise AttnError(n, "attn_timing_stop")
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split()
        out[name] = (int(cnt), float(ms))
    return out


def fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype) -> int:
    return int(lib().attn_fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype))


def bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype))


def bwd_fused_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype) -> int:
    return int(lib().attn_bwd_fused_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dtype))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# Pointer alignment the library requires (include/attn.h): 4 bytes for lse and
# the FP8 scale arrays, 16 bytes for every other tensor and the workspace.
_ALIGN4 = {"lse", "scales", "q_scales", "k_scales", "vt_scales"}


def _check(t, name: str):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    align = 4 if name in _ALIGN4 else 16
    if t.data_ptr() % align != 0:
        raise ValueError(f"{name} must start at a {align}-byte aligned address (a view with an odd "
                         "storage offset is not)")


def _want(t, shape, dtype, name: str):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must have shape {tuple(shape)} and dtype {dtype}, "
                         f"got {tuple(t.shape)} {t.dtype}")


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def fwd(q, k, v, *, causal: int = 0, scale: Optional[float] = None, out=None, lse=None,
        need_lse: bool = True, workspace=None, stream=None) -> Tuple["object", "object"]:
    """O (and lse) for q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] on the GPU.

    Returns (o, lse); lse is None when ``need_lse`` is False and no buffer was
    given. ``causal``: 0 none, 1 top-left, 2 bottom-right.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse"), (workspace, "workspace")):
        _check(t, n)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    dt = _dtype_code(q)
    _want(k, (B, Hkv, Sk, d), q.dtype, "k")
    _want(v, (B, Hkv, Sk, d), q.dtype, "v")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and need_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    ws_n = fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, dt)
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                        causal, sc, dt, _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def fwd_noalloc(q, k, v, out, lse=None, *, causal: int = 0, scale: Optional[float] = None, stream=None):
    """attn_fwd_noalloc: the forward into caller-given ``out`` (and ``lse``, or
    None) with the library's static scratch instead of a workspace; the
    library allocates nothing. Calls that overlap on one GPU race on that
    scratch."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse")):
        _check(t, n)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    dt = _dtype_code(q)
    _want(k, (B, Hkv, Sk, d), q.dtype, "k")
    _want(v, (B, Hkv, Sk, d), q.dtype, "v")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    st = lib().attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d, causal,
                                sc, dt, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_noalloc")
    return out, lse


def bwd(q, k, v, o, lse, dout, *, causal: int = 0, scale: Optional[float] = None, dq=None, dk=None,
        dv=None, workspace=None, stream=None, fused: bool = False):
    """(dq, dk, dv) for the forward that produced o and lse (bf16 only).

    The default is the two-pass backward (attn_bwd), the same bits on every
    run; ``fused=True`` runs the single pass with atomically accumulated dQ
    (attn_bwd_fused), slower on MI355X and kept for comparison."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (dout, "dout"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace")):
        _check(t, n)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    dt = _dtype_code(q)
    for t, n, shp in ((k, "k", k.shape), (v, "v", k.shape), (o, "o", q.shape), (dout, "dout", q.shape),
                      (dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _want(t, shp, q.dtype, n)
    _want(v, (B, Hkv, Sk, d), q.dtype, "v")
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_n = (bwd_fused_workspace_bytes if fused else bwd_workspace_bytes)(B, Hq, Hkv, Sq, Sk, d, causal, dt)
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib().attn_bwd_fused if fused else lib().attn_bwd
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), B, Hq, Hkv, Sq, Sk, d, causal, sc, dt, _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_fused" if fused else "attn_bwd")
    return dq, dk, dv


def _cu_array(cu, name: str):
    """A host ctypes int array from a sequence or CPU tensor of B+1 offsets."""
    vals = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    if len(vals) < 2:
        raise ValueError(f"{name} needs at least 2 entries (B+1 offsets), got {len(vals)}")
    return (ctypes.c_int * len(vals))(*vals), vals


def _varlen_cu(cu_seqlens_q, cu_seqlens_k):
    cq, vq = _cu_array(cu_seqlens_q, "cu_seqlens_q")
    ck, vk = _cu_array(cu_seqlens_k, "cu_seqlens_k")
    if len(vq) != len(vk):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    return cq, ck, len(vq) - 1, vq[-1], vk[-1]


def fwd_varlen_workspace_bytes(cu_seqlens_q, cu_seqlens_k, Hq, Hkv, d, causal, dtype) -> int:
    cq, ck, B, _, _ = _varlen_cu(cu_seqlens_q, cu_seqlens_k)
    return int(lib().attn_fwd_varlen_workspace_bytes(cq, ck, B, Hq, Hkv, d, causal, dtype))


def bwd_varlen_workspace_bytes(cu_seqlens_q, cu_seqlens_k, Hq, Hkv, d, causal, dtype) -> int:
    cq, ck, B, _, _ = _varlen_cu(cu_seqlens_q, cu_seqlens_k)
    return int(lib().attn_bwd_varlen_workspace_bytes(cq, ck, B, Hq, Hkv, d, causal, dtype))


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: int = 0, scale: Optional[float] = None,
               out=None, lse=None, need_lse: bool = True, workspace=None, stream=None):
    """O (and lse) for a packed batch of sequences of different lengths.

    q is [Hq, total_q, d], k and v [Hkv, total_k, d], head-major and packed:
    sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and rows
    cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v. The offsets are host
    data (a list or CPU tensor of B+1 ints). Returns (o [Hq, total_q, d],
    lse [Hq, total_q]).
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse"), (workspace, "workspace")):
        _check(t, n)
    cq, ck, B, tq, tk = _varlen_cu(cu_seqlens_q, cu_seqlens_k)
    Hq, _, d = q.shape
    Hkv = k.shape[0]
    dt = _dtype_code(q)
    _want(q, (Hq, tq, d), q.dtype, "q")
    _want(k, (Hkv, tk, d), q.dtype, "k")
    _want(v, (Hkv, tk, d), q.dtype, "v")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (Hq, tq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and need_lse:
        lse = torch.empty((Hq, tq), dtype=torch.float32, device=q.device)
    ws_n = int(lib().attn_fwd_varlen_workspace_bytes(cq, ck, B, Hq, Hkv, d, causal, dt))
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), cq, ck, B, Hq, Hkv,
                               d, causal, sc, dt, _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_varlen")
    return out, lse


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, *, causal: int = 0,
               scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv) of a packed batch, in the layout of fwd_varlen (bf16 only)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (dout, "dout"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace")):
        _check(t, n)
    cq, ck, B, tq, tk = _varlen_cu(cu_seqlens_q, cu_seqlens_k)
    Hq, _, d = q.shape
    Hkv = k.shape[0]
    dt = _dtype_code(q)
    qs, ks = (Hq, tq, d), (Hkv, tk, d)
    for t, n, shp in ((q, "q", qs), (k, "k", ks), (v, "v", ks), (o, "o", qs), (dout, "dout", qs),
                      (dq, "dq", qs), (dk, "dk", ks), (dv, "dv", ks)):
        _want(t, shp, q.dtype, n)
    _want(lse, (Hq, tq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_n = int(lib().attn_bwd_varlen_workspace_bytes(cq, ck, B, Hq, Hkv, d, causal, dt))
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                               _ptr(dk), _ptr(dv), cq, ck, B, Hq, Hkv, d, causal, sc, dt,
                               _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_varlen")
    return dq, dk, dv


def fwd_dropout(q, k, v, *, dropout_p: float, seed: int, offset: int = 0, causal: int = 0,
                scale: Optional[float] = None, out=None, lse=None, stream=None):
    """O and lse with dropout on the probabilities (bf16, [B, H, S, d]).

    The keep mask is a function of (seed, offset, batch, head, query, key)
    only, so bwd_dropout with the same arguments regenerates it.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (lse, "lse")):
        _check(t, n)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    _want(k, (B, Hkv, Sk, d), torch.bfloat16, "k")
    _want(v, (B, Hkv, Sk, d), torch.bfloat16, "v")
    _want(q, q.shape, torch.bfloat16, "q")
    _want(out, q.shape, q.dtype, "out")
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if lse is None else lse
    st = lib().attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d, causal,
                                sc, float(dropout_p), int(seed), int(offset), _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_dropout")
    return out, lse


def bwd_dropout(q, k, v, o, lse, dout, *, dropout_p: float, seed: int, offset: int = 0, causal: int = 0,
                scale: Optional[float] = None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv) of the forward that fwd_dropout computed with the same
    dropout_p, seed and offset."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (dout, "dout"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv"), (workspace, "workspace")):
        _check(t, n)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    for t, n, shp in ((q, "q", q.shape), (k, "k", k.shape), (v, "v", k.shape), (o, "o", q.shape),
                      (dout, "dout", q.shape), (dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _want(t, shp, torch.bfloat16, n)
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_n = bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal, ATTN_BF16)
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), B, Hq, Hkv, Sq, Sk, d, causal, sc, float(dropout_p), int(seed),
                                int(offset), _ptr(workspace), ws_bytes, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_bwd_dropout")
    return dq, dk, dv


def dropout_mask(B: int, Hq: int, Sq: int, Sk: int, *, dropout_p: float, seed: int, offset: int = 0,
                 device="cuda", stream=None):
    """The keep mask [B, Hq, Sq, Sk] (uint8, 1 = kept) the kernels regenerate."""
    import torch
    keep = torch.empty((B, Hq, Sq, Sk), dtype=torch.uint8, device=device)
    st = lib().attn_dropout_mask(_ptr(keep), B, Hq, Sq, Sk, float(dropout_p), int(seed), int(offset),
                                 _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_dropout_mask")
    return keep


def fp8_padded_keys(Sk: int) -> int:
    """Keys of the transposed FP8 V: Sk rounded up to a multiple of 64."""
    n = int(lib().attn_fp8_padded_keys(int(Sk)))
    if n < 0:
        raise AttnError(n, "attn_fp8_padded_keys")
    return n


def mxfp8_quantize_rows(x, *, codes=None, scales=None, stream=None):
    """bf16 [..., d] -> (E4M3 codes uint8 [..., d], E8M0 scales uint8 [..., d/32])."""
    import torch
    _check(x, "x")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], d // 32), dtype=torch.uint8, device=x.device)
    _check(codes, "codes")
    _check(scales, "scales")
    _want(codes, x.shape, torch.uint8, "codes")
    _want(scales, (*x.shape[:-1], d // 32), torch.uint8, "scales")
    st = lib().attn_mxfp8_quantize_rows(_ptr(x), _ptr(codes), _ptr(scales), rows, d, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_mxfp8_quantize_rows")
    return codes, scales


def mxfp8_quantize_vt(v, *, stream=None):
    """bf16 V [B, Hkv, Sk, d] -> (V^T codes tiled by 64 keys, uint8
    [B, Hkv, Skp/64, d, 64], scales uint8 [B, Hkv, Skp/64, d, 2]),
    Skp = fp8_padded_keys(Sk)."""
    import torch
    _check(v, "v")
    if v.dtype != torch.bfloat16:
        raise TypeError("v must be bfloat16")
    B, H, Sk, d = v.shape
    skp = fp8_padded_keys(Sk)
    codes = torch.empty((B, H, skp // 64, d, 64), dtype=torch.uint8, device=v.device)
    scales = torch.empty((B, H, skp // 64, d, 2), dtype=torch.uint8, device=v.device)
    st = lib().attn_mxfp8_quantize_vt(_ptr(v), _ptr(codes), _ptr(scales), B * H, Sk, d, _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_mxfp8_quantize_vt")
    return codes, scales


def fwd_fp8_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal) -> int:
    return int(lib().attn_fwd_fp8_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal))


def fwd_fp8(q8, q_scales, k8, k_scales, vt8, vt_scales, *, causal: int = 0, scale: Optional[float] = None,
            out=None, lse=None, need_lse: bool = True, workspace=None, stream=None):
    """Forward on MXFP8 operands (as the two quantisers give them): returns
    (o bf16 [B, Hq, Sq, d], lse float32 [B, Hq, Sq] or None)."""
    import torch
    for t, n in ((q8, "q8"), (q_scales, "q_scales"), (k8, "k8"), (k_scales, "k_scales"), (vt8, "vt8"),
                 (vt_scales, "vt_scales"), (out, "out"), (lse, "lse"), (workspace, "workspace")):
        _check(t, n)
    B, Hq, Sq, d = q8.shape
    _, Hkv, Sk, _ = k8.shape
    skp = fp8_padded_keys(Sk)
    u8 = torch.uint8
    _want(q8, (B, Hq, Sq, d), u8, "q8")
    _want(q_scales, (B, Hq, Sq, d // 32), u8, "q_scales")
    _want(k8, (B, Hkv, Sk, d), u8, "k8")
    _want(k_scales, (B, Hkv, Sk, d // 32), u8, "k_scales")
    _want(vt8, (B, Hkv, skp // 64, d, 64), u8, "vt8")
    _want(vt_scales, (B, Hkv, skp // 64, d, 2), u8, "vt_scales")
    _want(out, (B, Hq, Sq, d), torch.bfloat16, "out")
    _want(lse, (B, Hq, Sq), torch.float32, "lse")
    sc = float(scale) if scale is not None else 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None and need_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    ws_n = fwd_fp8_workspace_bytes(B, Hq, Hkv, Sq, Sk, d, causal)
    if workspace is None and ws_n > 0:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=q8.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().attn_fwd_fp8(_ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales), _ptr(vt8), _ptr(vt_scales),
                            _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d, causal, sc, _ptr(workspace), ws_bytes,
                            _stream(stream))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return out, lse
