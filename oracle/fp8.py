"""FP8 (MXFP8) attention inputs and their attention -- test infrastructure only.

[P1] §2.2 says FA3 runs attention in FP8, at twice the bf16 matrix rate, and
keeps it accurate by quantising block by block. The page fixes neither the
8-bit format nor the blocks. Readings taken (all listed in the design notes):

* Element format: OCP FP8 E4M3 ("OCP 8-bit Floating Point Specification",
  v1.0): one sign bit, four exponent bits with bias 7, three mantissa bits;
  exponent field 0 holds the subnormals m/8 * 2^-6; the code S.1111.111 is
  NaN, so the largest finite magnitude is 448 (S.1111.110). No infinities.
* Blocks: 32 consecutive elements share one power-of-two scale stored as an
  E8M0 byte (scale = 2^(byte - 127)), as in the OCP Microscaling (MX) v1.0
  format. Q and K are blocked along the head dimension (32 channels of one
  row); V along the keys (32 keys of one channel), because its block scale
  must apply to the operand that the P V product sums over.
* Scale choice: the smallest power of two 2^e with amax <= 448 * 2^e, so no
  element saturates (the MX specification's own rule, 2^(floor(log2 amax) -
  8), may clip values above 448); an all-zero block takes e = 0. e is
  clamped to the E8M0 range [-127, 127].
* Element rounding: round to nearest, ties to even, of x / 2^e (exact in any
  binary format, since 2^e is a power of two).
* FP8 attention is exact attention of the dequantised inputs: the oracle
  dequantises and calls the float64 definition.

The storage layouts are plain arrays here (codes and scale bytes in the
natural row-major order of the blocked axis); tests rearrange them into the
library's layouts.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .attention import attention_forward

__all__ = [
    "E4M3_MAX", "MX_BLOCK", "e4m3_decode", "e4m3_encode", "mx_block_exponent",
    "mx_quantize", "mx_dequantize", "attention_forward_fp8",
]

E4M3_MAX = 448.0
MX_BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    val = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0))
    val = np.where((ex == 0xF) & ((c & 0x7) == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each value, rounding to nearest with ties to even.

    Values must be finite with |x| <= 448 (the quantiser never produces more;
    anything else raises). Negative zero encodes as 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all() or (np.abs(x) > E4M3_MAX).any():
        raise ValueError("e4m3_encode takes finite values of magnitude <= 448")
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0x00)
    # exponent of the binade: 2^E <= a < 2^(E+1), floored at the subnormal binade
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # guard against log2 rounding at exact powers of two
    E = np.where(np.exp2(E) > a, E - 1, E)
    E = np.where(np.exp2(E + 1) <= a, E + 1, E)
    E = np.maximum(E, -6.0)                         # below 2^-6: subnormal spacing 2^-9
    step = np.exp2(E - 3.0)                         # spacing of the binade (3 mantissa bits)
    q = np.rint(a / step)                           # numpy rint: ties to even; a / step is exact
    # q counts steps: 8..16 in a normal binade (16 carries into the next), 0..8 subnormal
    carry = q >= 16
    E = np.where(carry, E + 1, E)
    q = np.where(carry, q / 2, q)
    normal = q >= 8
    field_e = np.where(normal, E + 7, 0).astype(np.int64)
    field_m = np.where(normal, q - 8, q).astype(np.int64)
    return (sign | (field_e << 3) | field_m).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """The smallest integer e with amax <= 448 * 2^e (0 for amax = 0),
    clamped to [-127, 127]. Exact: with amax = f 2^E, f in [0.5, 1) (frexp)
    and 448 = 0.875 * 2^9, the condition is f 2^E <= 0.875 2^(9 + e)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape, dtype=np.int64)
    flat_a, flat_o = amax.reshape(-1), out.reshape(-1)
    for i, a in enumerate(flat_a):
        if a == 0.0:
            flat_o[i] = 0
            continue
        f, E = math.frexp(float(a))
        e = E - 9 + (1 if f > 0.875 else 0)
        flat_o[i] = min(127, max(-127, e))
    return out


def mx_quantize(x, axis: int = -1) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantisation along ``axis`` (its length a multiple of 32).

    Returns (codes uint8 with x's shape, scale bytes uint8 with that axis
    divided by 32). Scale byte = e + 127 for the block exponent e of
    ``mx_block_exponent``; element code = RNE_e4m3(x / 2^e).
    """
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % MX_BLOCK:
        raise ValueError(f"blocked axis length {n} is not a multiple of {MX_BLOCK}")
    blocks = xm.reshape(*xm.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    e = mx_block_exponent(np.abs(blocks).max(axis=-1))
    codes = e4m3_encode(blocks / np.exp2(e.astype(np.float64))[..., None])
    codes = np.moveaxis(codes.reshape(xm.shape), -1, axis)
    scales = np.moveaxis((e + 127).astype(np.uint8), -1, axis)
    return codes, scales


def mx_dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """Values code * 2^(scale byte - 127), blocks of 32 along ``axis``."""
    cm = np.moveaxis(np.asarray(codes), axis, -1)
    sm = np.moveaxis(np.asarray(scales), axis, -1)
    n = cm.shape[-1]
    vals = e4m3_decode(cm).reshape(*cm.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    vals = vals * np.exp2(sm.astype(np.float64) - 127.0)[..., None]
    return np.moveaxis(vals.reshape(cm.shape), -1, axis)


def attention_forward_fp8(q8, qs, k8, ks, vt8, vs, *, causal: int = 0, scale: Optional[float] = None,
                          rows=None, Sq: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of MXFP8 inputs: dequantise, then the float64 definition.

    q8 [B, Hq, Sq, d], qs [B, Hq, Sq, d/32]; k8 [B, Hkv, Sk, d], ks
    [B, Hkv, Sk, d/32]; vt8 [B, Hkv, d, Skp] (V transposed, keys padded to a
    multiple of 32), vs [B, Hkv, d, Skp/32]. Only the first Sk = k8.shape[2]
    keys of V take part. ``rows``/``Sq`` as in attention_forward.
    """
    q = mx_dequantize(q8, qs, axis=-1)
    k = mx_dequantize(k8, ks, axis=-1)
    Sk = k.shape[2]
    v = np.swapaxes(mx_dequantize(vt8, vs, axis=-1), -1, -2)[:, :, :Sk, :]
    return attention_forward(q, k, v, causal=causal, scale=scale, rows=rows, Sq=Sq)
