"""Pins for the MXFP8 part of the oracle (CPU only): the E4M3 code table
against the OCP specification's printed values and torch's float8_e4m3fn
conversion (a library routine), brute force for the block exponent, error
bounds of the quantiser, and exactness on inputs the format represents."""
import math

import numpy as np
import pytest
import torch

from oracle import attention_forward
from oracle import fp8


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------ E4M3 codes
def test_decode_specification_values():
    # values the OCP FP8 specification states for E4M3
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x77: 240.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in table.items():
        assert fp8.e4m3_decode(c) == v, hex(c)
    assert np.isnan(fp8.e4m3_decode(0x7F)) and np.isnan(fp8.e4m3_decode(0xFF))
    assert np.signbit(fp8.e4m3_decode(0x80)) and fp8.e4m3_decode(0x80) == 0.0


def test_decode_matches_torch_for_every_code():
    c = np.arange(256, dtype=np.uint8)
    d, t = fp8.e4m3_decode(c), _torch_decode(c)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    ok = ~np.isnan(d)
    assert np.array_equal(d[ok], t[ok])


def test_encode_round_trips_every_finite_code():
    c = np.arange(256, dtype=np.uint8)
    d = fp8.e4m3_decode(c)
    ok = ~np.isnan(d)
    assert np.array_equal(fp8.e4m3_encode(d[ok]), c[ok])


def test_encode_ties_go_to_even_and_match_torch():
    c = np.arange(0x00, 0x7F, dtype=np.uint8)            # non-negative finite codes, ascending
    d = fp8.e4m3_decode(c)
    mids = (d[:-1] + d[1:]) / 2
    enc = fp8.e4m3_encode(mids)
    # of the two neighbours, the tie goes to the one with an even mantissa field
    lo, hi = c[:-1], c[1:]
    want = np.where((lo & 1) == 0, lo, hi)
    assert np.array_equal(enc, want)
    assert np.array_equal(enc, _torch_encode(mids))
    assert np.array_equal(fp8.e4m3_encode(-mids), _torch_encode(-mids))


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000), rng.standard_normal(2000) * 1e-3])
    x = np.clip(x, -448, 448)
    assert np.array_equal(fp8.e4m3_encode(x), _torch_encode(x))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode([449.0])
    with pytest.raises(ValueError):
        fp8.e4m3_encode([np.nan])


# ------------------------------------------------------------- block exponent
def test_block_exponent_brute_force():
    rng = np.random.default_rng(1)
    amax = np.concatenate([np.exp2(rng.uniform(-40, 40, 3000)), 448.0 * np.exp2(np.arange(-20, 21)),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 21)), np.inf),
                           np.nextafter(448.0 * np.exp2(np.arange(-20, 21)), 0), [1.0, 0.875, 224.0]])
    got = fp8.mx_block_exponent(amax)
    for a, e in zip(amax, got):
        brute = next(x for x in range(-150, 150) if a <= 448.0 * 2.0 ** x)
        assert e == max(-127, min(127, brute)), a
    assert fp8.mx_block_exponent(0.0) == 0


# ------------------------------------------------------------------ quantiser
def test_quantize_bounds_and_zero_block():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 128)) * np.exp2(rng.integers(-8, 9, (3, 5, 1)))
    x[0, 0, :32] = 0.0
    codes, scales = fp8.mx_quantize(x, axis=-1)
    assert codes.shape == x.shape and scales.shape == (3, 5, 4)
    assert scales[0, 0, 0] == 127 and (codes[0, 0, :32] == 0).all()
    vals = fp8.e4m3_decode(codes)
    blocks = np.abs(vals).reshape(3, 5, 4, 32).max(axis=-1)
    nz = np.abs(x).reshape(3, 5, 4, 32).max(axis=-1) > 0
    # the block max lands in the top binade or the one below it (no waste, no saturation)
    assert (blocks[nz] <= 448.0).all() and (blocks[nz] >= 224.0 * (1 - 2.0 ** -4)).all()
    deq = fp8.mx_dequantize(codes, scales, axis=-1)
    s = np.exp2(scales.astype(np.float64) - 127).repeat(32, axis=-1)
    # round to nearest: at most half a step of the element's binade (subnormal step 2^-9)
    a = np.abs(x) / s
    step = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6) - 3)
    assert (np.abs(deq - x) <= 0.5 * step * s * (1 + 1e-12)).all()


def test_quantize_is_exact_on_representable_blocks_along_any_axis():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, (2, 64, 96)).astype(np.uint8)
    codes[..., ::32] = 0x7E                              # every block holds +448, so e is its own
    e = rng.integers(-10, 11, (2, 64, 3))
    x = fp8.e4m3_decode(codes) * np.exp2(e.astype(np.float64)).repeat(32, axis=-1)
    c2, s2 = fp8.mx_quantize(x, axis=-1)
    assert np.array_equal(c2, codes) and np.array_equal(s2.astype(np.int64), e + 127)
    xt = np.swapaxes(x, 1, 2)
    c3, s3 = fp8.mx_quantize(xt, axis=1)
    assert c3.shape == xt.shape and s3.shape == (2, 3, 64)
    assert np.array_equal(fp8.mx_dequantize(c3, s3, axis=1), xt)


# ------------------------------------------------------------- FP8 attention
def test_fp8_attention_is_attention_of_dequantised_inputs():
    """On inputs the format represents exactly, FP8 attention equals the
    float64 definition on the original values; keys past Sk in the padded
    V^T take no part."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, Sq, Sk, d, Skp = 1, 4, 2, 40, 50, 64, 64

    def representable(shape, axis):
        c = rng.integers(0, 0x7F, shape).astype(np.uint8) | (rng.integers(0, 2, shape).astype(np.uint8) << 7)
        e = rng.integers(-9, -5, shape[:axis] + (shape[axis] // 32,) + shape[axis + 1:])
        x = fp8.e4m3_decode(c) * np.exp2(np.repeat(e.astype(np.float64), 32, axis=axis))
        return x

    q = representable((B, Hq, Sq, d), 3)
    k = representable((B, Hkv, Sk, d), 3)
    vt = representable((B, Hkv, d, Skp), 3)
    q8, qs = fp8.mx_quantize(q)
    k8, ks = fp8.mx_quantize(k)
    v8, vs = fp8.mx_quantize(vt)
    v8[..., Sk:] = 0x7E                                   # garbage in the padding keys
    for causal in (0, 1, 2):
        o, lse = fp8.attention_forward_fp8(q8, qs, k8, ks, v8, vs, causal=causal, scale=0.125)
        o_ref, lse_ref = attention_forward(q, k, np.swapaxes(vt, -1, -2)[:, :, :Sk], causal=causal, scale=0.125)
        assert np.array_equal(lse, lse_ref)
        assert np.array_equal(o, o_ref)
