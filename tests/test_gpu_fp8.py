"""FP8 (MXFP8) forward parity on the GPU: the quantisers bit for bit against
the oracle's, and the FP8 forward against exact attention of the oracle's
own dequantised inputs.

Tolerance of O, derived from the kernel's arithmetic: the score product and
the softmax run in fp32 on the exact input values, and the only coarse step
is rounding each probability to E4M3 before the P V product. The kernel forms
P' = 2^6 2^(s - m') with a reference max m' within 2 (log2) below the row
max, so P' <= 2^8 and every P' of the E4M3 normal range carries a relative
error of at most 2^-4, every smaller one an absolute error of at most 2^-10
(half the subnormal spacing). The denominator l' = sum P' (fp32, unrounded)
is at least 2^6 L with L = sum_j exp(s_j - max_j s_j). Hence, per element,

  |o - o_ref| <= 2^-4 sum_j p_j |v_jc| + 2^-16 sum_j |v_jc| / L
                 + 2^-8 |o_ref| (bf16 output) + 1e-5 (fp32 sums),

summed over the visible keys j. The test also checks the relative Frobenius
error per head, a statistical check: the rounding errors of different keys are
independent, so it is close to the RMS relative error of E4M3 rounding, which
for mantissas m spread log-uniformly over [1, 2) is 2^-4 sqrt(E[m^-2] / 3) =
2^-4 sqrt(0.541 / 3) ~ 2.65 %; the bound is 1.5 times that, 4e-2 (observed
worst heads from 1.3 % to 3.1 % over the cases below; a head averages fewer
independent roundings when few keys dominate its rows, so its figure spreads
around the RMS value). lse does not depend on the rounding of P;
it moves by at most the largest score error, and a score is an fp32 dot
product of d exact products, which any summation order with directed
rounding keeps within d 2^-23 sum_c |q_c k_c| (= 2^-16 for d = 128). So
|lse - lse_ref| <= 1e-3 + 2^-16 scale max_j sum_c |q_ic k_jc|: 1e-3 for the
N(0, 1) rows, up to ~3e-3 for the rows scaled x30.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import fp8 as ofp8
from parity import assert_finite, rel_fro, to_device, to_host_f64

pytestmark = pytest.mark.gpu

FP8_REL_FRO = 4e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_38_amd as m
    m.lib()
    return m


def _u8(t):
    return t.cpu().numpy()


def _tile64(a):
    """[B, H, d, Skp] -> the library's [B, H, Skp/64, d, 64] (64-key tiles)."""
    B, H, d, n = a.shape
    return np.ascontiguousarray(a.reshape(B, H, d, n // 64, 64).transpose(0, 1, 3, 2, 4))


def _oracle_quant(q, k, v, Skp):
    """The oracle's MXFP8 operands (float64 inputs): Q and K codes and scales,
    V^T codes in the oracle's natural [B, H, d, Skp] and in the library's
    tiled layout, V^T scales in the library's [B, H, Skp/64, d, 2] and the
    natural [B, H, d, Skp/32]."""
    q8, qs = ofp8.mx_quantize(q, axis=-1)
    k8, ks = ofp8.mx_quantize(k, axis=-1)
    B, H, Sk, d = v.shape
    vt = np.zeros((B, H, d, Skp))
    vt[..., :Sk] = np.swapaxes(v, -1, -2)
    vt8, vts_nat = ofp8.mx_quantize(vt, axis=-1)                 # scales [B, H, d, Skp/32]
    vts = vts_nat.reshape(B, H, d, Skp // 64, 2).transpose(0, 1, 3, 2, 4)
    return q8, qs, k8, ks, vt8, np.ascontiguousarray(vts), vts_nat


def _fp8_tolerance(q, k, v, causal, scale, rows=None, Sq=None):
    """Per-element bound of the module docstring (float64 dequantised inputs)."""
    B, Hq, n, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    Sq_ = n if Sq is None else Sq
    vis = oracle.visible_mask(Sq_, Sk, causal, rows)
    a_abs, _ = oracle.attention_forward(q, k, np.abs(v), causal=causal, scale=scale, rows=rows, Sq=Sq)
    tail = np.zeros((B, Hq, n, d))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // g].T)
            s = np.where(vis, s, -np.inf)
            mx = s.max(axis=1, initial=-np.inf)
            ok = np.isfinite(mx)
            L = np.ones(n)
            L[ok] = np.exp(s[ok] - mx[ok, None]).sum(axis=1)
            tail[b, h] = (vis.astype(np.float64) @ np.abs(v[b, h // g])) / L[:, None]
    return 2.0 ** -4 * a_abs + 2.0 ** -16 * tail


def _lse_tolerance(q, k, causal, scale, rows=None, Sq=None):
    """1e-3 + 2^-16 scale max_j sum_c |q_ic k_jc| per row (module docstring)."""
    B, Hq, n, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    vis = oracle.visible_mask(n if Sq is None else Sq, Sk, causal, rows)
    tol = np.full((B, Hq, n), 1e-3)
    for b in range(B):
        for h in range(Hq):
            a = np.abs(q[b, h]) @ np.abs(k[b, h // (Hq // Hkv)]).T
            tol[b, h] += 2.0 ** -16 * scale * np.where(vis, a, 0.0).max(axis=1, initial=0.0)
    return tol


def _check_fp8_lse(lse, lse_ref, tol):
    assert not np.isnan(lse).any() and not np.isposinf(lse).any()
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf), "lse = -inf exactly where no key is visible"
    err = np.abs(lse[~ninf] - lse_ref[~ninf])
    assert (err <= tol[~ninf]).all(), f"lse: {int((err > tol[~ninf]).sum())} rows outside the bound, worst {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def _check_fp8_o(o, o_ref, tol, what="O", statistical=True):
    """The per-element bound, and (statistical) the per-head relative
    Frobenius error, which assumes that many keys share each row's weight."""
    assert o.shape == o_ref.shape
    assert_finite(what, o)
    err = np.abs(o - o_ref)
    bound = tol + 2.0 ** -8 * np.abs(o_ref) + 1e-5
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements outside the FP8 bound; "
                           f"worst excess {(err - bound).max():.3e}")
    if not statistical:
        return float(err.max()) if err.size else 0.0
    per_head = [rel_fro(o[b, h], o_ref[b, h]) for b in range(o.shape[0]) for h in range(o.shape[1])
                if np.linalg.norm(o_ref[b, h]) > 0]
    worst = max(per_head) if per_head else 0.0
    assert worst <= FP8_REL_FRO, f"{what}: relative Frobenius error {worst:.3e} > {FP8_REL_FRO}"
    return worst


# ----------------------------------------------------------------- quantisers
QUANT = [(1, 2, 100, 1), (2, 3, 64, 2), (1, 1, 1, 3), (1, 4, 2000, 4), (2, 2, 31, 5)]


@pytest.mark.parametrize("B,H,S,seed", QUANT)
def test_quantize_rows_bit_exact(attn, B, H, S, seed):
    import torch
    _say(f"quantize rows B={B} H={H} S={S}")
    w = synth.Workload("fp8_rows", B, H, H, S, S, 128, "bf16", 0, seed=seed, outlier_frac=0.05,
                       outlier_scale=30.0)
    x = synth.make_inputs(w)
    xq = x["q"].copy()
    xq[0, 0, 0, :32] = 0                                   # an all-zero block
    xq[0, 0, 0, 32:64] = synth.bf16_bits_from_f32(np.full(32, 3.0e-38, np.float32))    # tiny values
    xq[0, -1, -1, 96:] = synth.bf16_bits_from_f32(np.linspace(-1e30, 1e30, 32).astype(np.float32))
    codes, scales = attn.mxfp8_quantize_rows(to_device(xq, "bf16"))
    torch.cuda.synchronize()
    c_ref, s_ref = ofp8.mx_quantize(synth.to_f64(xq, "bf16"), axis=-1)
    assert np.array_equal(_u8(scales), s_ref)
    assert np.array_equal(_u8(codes), c_ref), f"{int((_u8(codes) != c_ref).sum())} codes differ"


# The V^T quantiser runs at most 2048 workgroups that stride over the (head,
# 64-key tile) units: exactly 2048 units, 2079 (the first 31 workgroups take a
# second unit) and the long-context benchmark's 8192 (four each).
QUANT_VT = QUANT + [(1, 32, 4096, 6), (3, 11, 4000, 7), (2, 32, 8192, 8)]


@pytest.mark.parametrize("B,H,S,seed", QUANT_VT)
def test_quantize_vt_bit_exact(attn, B, H, S, seed):
    import torch
    _say(f"quantize V^T B={B} H={H} Sk={S}")
    w = synth.Workload("fp8_vt", B, H, H, S, S, 128, "bf16", 0, seed=seed)
    x = synth.make_inputs(w)
    xv = x["v"].copy()
    xv[..., :1, :] = 0                                     # key 0 zero in every channel
    codes, scales = attn.mxfp8_quantize_vt(to_device(xv, "bf16"))
    torch.cuda.synchronize()
    Skp = attn.fp8_padded_keys(S)
    v = synth.to_f64(xv, "bf16")
    _, _, _, _, vt8, vts, _ = _oracle_quant(np.zeros((1, 1, 1, 128)), np.zeros((1, 1, 1, 128)), v, Skp)
    assert np.array_equal(_u8(scales), vts)
    vt8 = _tile64(vt8)
    assert np.array_equal(_u8(codes), vt8), f"{int((_u8(codes) != vt8).sum())} codes differ"


# ---------------------------------------------------------------- FP8 forward
FWD = [
    # B, Hq, Hkv, Sq, Sk, causal, seed      several tiles with ragged tails
    (1, 2, 2, 256, 256, 0, 11),
    (1, 2, 2, 300, 300, 1, 12),
    (2, 4, 2, 257, 333, 2, 13),
    (1, 8, 2, 200, 77, 2, 14),       # Sq > Sk, bottom-right: the first 123 rows see no key
    (1, 4, 1, 130, 520, 1, 15),      # top-left with Sk > Sq: keys >= 130 never visible
    (1, 6, 2, 100, 100, 0, 16),      # 3 query heads per KV head
    (1, 32, 8, 64, 2000, 0, 17),     # 4 query heads per KV head, ragged 2000 keys
    (1, 4, 4, 1, 700, 0, 18),        # one query row (split-key decode)
    (1, 2, 2, 64, 64, 1, 19),        # exactly one tile
    # split-key decode shapes (Hq/Hkv * Sq <= 32)
    (2, 8, 2, 1, 1000, 0, 31),       # 4 query heads per KV head, one row each
    (1, 32, 1, 1, 5000, 0, 32),      # 32 query heads share one KV head
    (1, 4, 4, 3, 700, 2, 33),        # 3 rows per head, bottom-right mask
    (3, 2, 1, 16, 2049, 1, 34),      # 32 packed rows, top-left mask, ragged keys
    (1, 4, 1, 2, 64, 0, 35),         # a single key tile
    (1, 8, 2, 1, 30, 0, 36),         # fewer keys than one tile
]


def _fwd_case(attn, B, Hq, Hkv, Sq, Sk, causal, seed, outliers=0.0):
    import torch
    w = synth.Workload("fp8_fwd", B, Hq, Hkv, Sq, Sk, 128, "bf16", causal, seed=seed,
                       outlier_frac=outliers, outlier_scale=30.0)
    x = synth.make_inputs(w)
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v")}
    Skp = attn.fp8_padded_keys(Sk)
    q8, qs, k8, ks, vt8, vts, vts_nat = _oracle_quant(f["q"], f["k"], f["v"], Skp)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q8, qs, k8, ks, _tile64(vt8), vts)]
    o, lse = attn.fwd_fp8(*dev, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ofp8.attention_forward_fp8(q8, qs, k8, ks, vt8, vts_nat, causal=causal, scale=w.scale)
    qd = ofp8.mx_dequantize(q8, qs)
    kd = ofp8.mx_dequantize(k8, ks)
    vd = np.swapaxes(ofp8.mx_dequantize(vt8, vts_nat), -1, -2)[:, :, :Sk]
    tol = _fp8_tolerance(qd, kd, vd, causal, w.scale)
    ltol = _lse_tolerance(qd, kd, causal, w.scale)
    return to_host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, tol, ltol


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal,seed", FWD)
def test_fwd_fp8_matches_oracle(attn, B, Hq, Hkv, Sq, Sk, causal, seed):
    _say(f"fwd_fp8 B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} causal={causal}")
    o, lse, o_ref, lse_ref, tol, ltol = _fwd_case(attn, B, Hq, Hkv, Sq, Sk, causal, seed)
    fro = _check_fp8_o(o, o_ref, tol)
    le = _check_fp8_lse(lse, lse_ref, ltol)
    _say(f"  relative Frobenius error (worst head) {fro:.3e}, lse max err {le:.3e}")


def _random_fwd_shapes(n=8, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 8, 16]))
        Sq = 1 if i % 4 == 2 else int(rng.integers(2, 500))
        out.append((int(rng.integers(1, 3)), Hkv * g, Hkv, Sq, int(rng.integers(1, 900)), int(rng.integers(0, 3)),
                    600 + i))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal,seed", _random_fwd_shapes())
def test_fwd_fp8_random_shapes(attn, B, Hq, Hkv, Sq, Sk, causal, seed):
    """Seeded random shapes (fixed seed: the same ones every run), prefill and
    split-key decode, all mask modes, against the oracle's MXFP8 forward."""
    _say(f"fwd_fp8 random B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} causal={causal}")
    o, lse, o_ref, lse_ref, tol, ltol = _fwd_case(attn, B, Hq, Hkv, Sq, Sk, causal, seed)
    fro = _check_fp8_o(o, o_ref, tol)
    le = _check_fp8_lse(lse, lse_ref, ltol)
    _say(f"  relative Frobenius error (worst head) {fro:.3e}, lse max err {le:.3e}")


def test_fwd_fp8_outlier_rows(attn):
    """Rows scaled x30 push the scores far past exp's range; the per-block
    scales absorb the magnitude and the recurrence stays finite."""
    _say("fwd_fp8 outlier rows")
    o, lse, o_ref, lse_ref, tol, ltol = _fwd_case(attn, 1, 4, 4, 600, 600, 1, 21, outliers=0.05)
    assert np.isfinite(lse_ref).all() and lse_ref.max() > 88.8
    fro = _check_fp8_o(o, o_ref, tol)
    le = _check_fp8_lse(lse, lse_ref, ltol)
    _say(f"  relative Frobenius error (worst head) {fro:.3e}, lse max err {le:.3e} "
         f"(bound on that row {ltol.reshape(-1)[np.argmax(np.abs(lse - lse_ref))]:.3e})")


@pytest.mark.parametrize("Sq,causal", [(520, 0), (520, 1), (1, 0)], ids=["prefill", "prefill_causal", "decode"])
def test_fwd_fp8_scores_growing_across_key_tiles(attn, Sq, causal):
    """Key tiles of growing norm (each 64-key tile x1.6) and a jump of about
    2^11 in the scores at the last tiles: the reference max moves at almost
    every tile and the probabilities against the old reference would overflow
    E4M3 by far, in the prefill and in the split-key decode."""
    import torch
    _say(f"fwd_fp8 growing scores Sq={Sq} causal={causal}")
    Sk = 520
    w = synth.Workload("fp8_growth", 1, 4, 4, Sq, Sk, 128, "bf16", causal, seed=4300 + Sq + causal)
    x = synth.make_inputs(w)
    tile = np.arange(Sk) // 64
    factor = 1.6 ** tile
    factor[tile >= 7] *= 12.0
    x["k"] = synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(x["k"]) * factor[None, None, :, None].astype(np.float32))
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v")}
    Skp = attn.fp8_padded_keys(Sk)
    q8, qs, k8, ks, vt8, vts, vts_nat = _oracle_quant(f["q"], f["k"], f["v"], Skp)
    dev = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q8, qs, k8, ks, _tile64(vt8), vts)]
    o, lse = attn.fwd_fp8(*dev, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ofp8.attention_forward_fp8(q8, qs, k8, ks, vt8, vts_nat, causal=causal, scale=w.scale)
    qd = ofp8.mx_dequantize(q8, qs)
    kd = ofp8.mx_dequantize(k8, ks)
    vd = np.swapaxes(ofp8.mx_dequantize(vt8, vts_nat), -1, -2)[:, :, :Sk]
    # one key dominates most rows here, so only the per-element bound applies
    worst = _check_fp8_o(to_host_f64(o), o_ref, _fp8_tolerance(qd, kd, vd, causal, w.scale), statistical=False)
    le = _check_fp8_lse(lse.cpu().numpy().astype(np.float64), lse_ref, _lse_tolerance(qd, kd, causal, w.scale))
    _say(f"  max abs error {worst:.3e}, lse max err {le:.3e}")


def test_fwd_fp8_empty_rows_and_no_keys(attn):
    import torch
    _say("fwd_fp8 no keys")
    z = torch.zeros((1, 2, 5, 128), dtype=torch.uint8, device="cuda")
    zs = torch.full((1, 2, 5, 4), 127, dtype=torch.uint8, device="cuda")
    k = torch.zeros((1, 2, 0, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((1, 2, 0, 4), dtype=torch.uint8, device="cuda")
    vt = torch.zeros((1, 2, 0, 128, 64), dtype=torch.uint8, device="cuda")
    vs = torch.zeros((1, 2, 0, 128, 2), dtype=torch.uint8, device="cuda")
    o, lse = attn.fwd_fp8(z, zs, k, ks, vt, vs, causal=0, scale=0.1)
    torch.cuda.synchronize()
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


def test_fwd_fp8_end_to_end_long_context_sampled(attn):
    """The long-context workload (B=2, H=32, S=8192, d=128, causal, 1% of
    rows x30) through the GPU quantisers and the FP8 forward, in the launch
    configuration the benchmark times; sampled rows of four heads (every one
    holding x30 rows) against the oracle's quantisation and FP8 attention of
    the same bf16 inputs."""
    import torch
    w = synth.get_workload("long_causal_d128")
    _say("fwd_fp8 long-context end to end (sampled)")
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    q8, qs = attn.mxfp8_quantize_rows(q)
    k8, ks = attn.mxfp8_quantize_rows(k)
    vt8, vts = attn.mxfp8_quantize_vt(v)
    o, lse = attn.fwd_fp8(q8, qs, k8, ks, vt8, vts, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert "fwd_fp8" in attn.last_dispatch()
    rng = np.random.default_rng(99)
    for b, h in ((0, 0), (0, 17), (1, 5), (1, 31)):
        out_rows = x["outlier_rows"][b, h]
        rows = np.unique(np.concatenate([[0, 1, 63, 64, 4095, w.Sq - 1], out_rows[:6],
                                         rng.choice(w.Sq, 10, replace=False)]))
        qf = synth.to_f64(x["q"][b:b + 1, h:h + 1], "bf16")
        kf = synth.to_f64(x["k"][b:b + 1, h:h + 1], "bf16")
        vf = synth.to_f64(x["v"][b:b + 1, h:h + 1], "bf16")
        q8r, qsr, k8r, ksr, vt8r, _, vtsr = _oracle_quant(qf[:, :, rows], kf, vf, w.Sk)
        o_ref, lse_ref = ofp8.attention_forward_fp8(q8r, qsr, k8r, ksr, vt8r, vtsr, causal=w.causal,
                                                    scale=w.scale, rows=rows, Sq=w.Sq)
        qd = ofp8.mx_dequantize(q8r, qsr)
        kd = ofp8.mx_dequantize(k8r, ksr)
        vd = np.swapaxes(ofp8.mx_dequantize(vt8r, vtsr), -1, -2)
        tol = _fp8_tolerance(qd, kd, vd, w.causal, w.scale, rows=rows, Sq=w.Sq)
        ltol = _lse_tolerance(qd, kd, w.causal, w.scale, rows=rows, Sq=w.Sq)
        og = to_host_f64(o[b:b + 1, h:h + 1, torch.from_numpy(rows).cuda()])
        lg = lse[b:b + 1, h:h + 1, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        err = np.abs(og - o_ref)
        bound = tol + 2.0 ** -8 * np.abs(o_ref) + 1e-5
        assert_finite("O", og)
        assert (err <= bound).all(), f"(b={b}, h={h}): {int((err > bound).sum())} elements outside the FP8 bound"
        _check_fp8_lse(lg, lse_ref, ltol)


def test_fwd_fp8_is_deterministic(attn):
    import torch
    _say("fwd_fp8 determinism")
    w = synth.Workload("fp8_det", 1, 8, 2, 700, 900, 128, "bf16", 1, seed=23)
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    ops = attn.mxfp8_quantize_rows(q) + attn.mxfp8_quantize_rows(k) + attn.mxfp8_quantize_vt(v)
    o1, l1 = attn.fwd_fp8(*ops, causal=1)
    o2, l2 = attn.fwd_fp8(*ops, causal=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_fp8_gqa_prefill_full_size_sampled(attn):
    """The GQA prefill workload (Hq=32, Hkv=8, S=4096, causal) through the
    GPU quantisers and the FP8 forward; sampled rows of one query head of
    every KV head against the oracle's quantisation and FP8 attention."""
    import torch
    w = synth.get_workload("gqa_prefill")
    _say("fwd_fp8 GQA prefill end to end (sampled)")
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    ops = attn.mxfp8_quantize_rows(q) + attn.mxfp8_quantize_rows(k) + attn.mxfp8_quantize_vt(v)
    o, lse = attn.fwd_fp8(*ops, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    g = w.Hq // w.Hkv
    for hk in range(w.Hkv):
        h = hk * g + int(rng.integers(g))
        rows = np.unique(np.concatenate([[0, 1, 255, 256, w.Sq - 1], rng.choice(w.Sq, 12, replace=False)]))
        qf = synth.to_f64(x["q"][:, h:h + 1], "bf16")
        kf = synth.to_f64(x["k"][:, hk:hk + 1], "bf16")
        vf = synth.to_f64(x["v"][:, hk:hk + 1], "bf16")
        q8r, qsr, k8r, ksr, vt8r, _, vtsr = _oracle_quant(qf[:, :, rows], kf, vf, w.Sk)
        o_ref, lse_ref = ofp8.attention_forward_fp8(q8r, qsr, k8r, ksr, vt8r, vtsr, causal=w.causal,
                                                    scale=w.scale, rows=rows, Sq=w.Sq)
        qd, kd = ofp8.mx_dequantize(q8r, qsr), ofp8.mx_dequantize(k8r, ksr)
        vd = np.swapaxes(ofp8.mx_dequantize(vt8r, vtsr), -1, -2)
        tol = _fp8_tolerance(qd, kd, vd, w.causal, w.scale, rows=rows, Sq=w.Sq)
        ltol = _lse_tolerance(qd, kd, w.causal, w.scale, rows=rows, Sq=w.Sq)
        idx = torch.from_numpy(rows).cuda()
        og = to_host_f64(o[:, h:h + 1, idx])
        lg = lse[:, h:h + 1, idx].cpu().numpy().astype(np.float64)
        err = np.abs(og - o_ref)
        bound = tol + 2.0 ** -8 * np.abs(o_ref) + 1e-5
        assert_finite("O", og)
        assert (err <= bound).all(), f"head {h}: {int((err > bound).sum())} elements outside the FP8 bound"
        _check_fp8_lse(lg, lse_ref, ltol)


def test_fwd_fp8_decode_full_size_sampled(attn):
    """The GQA decode workload (B=16, Hq=32, Hkv=8, one query row, 32768 keys)
    through the GPU quantisers and the FP8 split-key decode, in the launch
    configuration the benchmark times; every query head of four batches
    against the oracle's quantisation and FP8 attention."""
    import torch
    w = synth.get_workload("gqa_decode")
    _say("fwd_fp8 GQA decode end to end (sampled)")
    x = synth.make_inputs(w)
    q, k, v = (to_device(x[n], "bf16") for n in ("q", "k", "v"))
    ops = attn.mxfp8_quantize_rows(q) + attn.mxfp8_quantize_rows(k) + attn.mxfp8_quantize_vt(v)
    o, lse = attn.fwd_fp8(*ops, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert "fwd_fp8_split" in attn.last_dispatch()
    g = w.Hq // w.Hkv
    for b in (0, 5, 10, 15):
        for hk in range(w.Hkv):
            qf = synth.to_f64(x["q"][b:b + 1, hk * g:(hk + 1) * g], "bf16")
            kf = synth.to_f64(x["k"][b:b + 1, hk:hk + 1], "bf16")
            vf = synth.to_f64(x["v"][b:b + 1, hk:hk + 1], "bf16")
            q8r, qsr, k8r, ksr, vt8r, _, vtsr = _oracle_quant(qf, kf, vf, w.Sk)
            o_ref, lse_ref = ofp8.attention_forward_fp8(q8r, qsr, k8r, ksr, vt8r, vtsr, causal=0, scale=w.scale)
            qd, kd = ofp8.mx_dequantize(q8r, qsr), ofp8.mx_dequantize(k8r, ksr)
            vd = np.swapaxes(ofp8.mx_dequantize(vt8r, vtsr), -1, -2)
            tol = _fp8_tolerance(qd, kd, vd, 0, w.scale)
            ltol = _lse_tolerance(qd, kd, 0, w.scale)
            og = to_host_f64(o[b:b + 1, hk * g:(hk + 1) * g])
            lg = lse[b:b + 1, hk * g:(hk + 1) * g].cpu().numpy().astype(np.float64)
            err = np.abs(og - o_ref)
            bound = tol + 2.0 ** -8 * np.abs(o_ref) + 1e-5
            assert_finite("O", og)
            assert (err <= bound).all(), f"(b={b}, kv head {hk}): {int((err > bound).sum())} elements outside the bound"
            _check_fp8_lse(lg, lse_ref, ltol)


@pytest.mark.parametrize("Sq", [1, 64])
@pytest.mark.parametrize("path", ["bf16", "fp8"])
def test_maximum_key_count_closed_form(attn, path, Sq):
    """Sk = 2^24 - 1 keys (the largest the library accepts; a bf16 head of K
    or V is then 4 GiB minus 256 bytes, so every 32-bit byte offset is in
    use). With K = 0 every visible key has probability 1/Sk, so O is the mean
    of V and lse = ln(Sk). V is zero except value 1 in every channel of the
    last 100 keys and 2 more in channel 0 of the first 50: O[0] = 200/Sk,
    O[c > 0] = 100/Sk, exactly representable sums in fp32 (all below 2^24),
    and in E4M3 (1 and 3 times a power-of-two block scale). Sq = 1 runs the
    split-key decode kernels, Sq = 64 (256 grouped rows) the prefill ones."""
    import torch
    Sk = (1 << 24) - 1
    _say(f"Sq = {Sq}, Sk = {Sk} ({path})")
    B, Hq, Hkv, d = 1, 4, 1, 128
    q = torch.randn((B, Hq, Sq, d), device="cuda").to(torch.bfloat16)
    k = torch.zeros((B, Hkv, Sk, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, Hkv, Sk, d), dtype=torch.bfloat16, device="cuda")
    v[:, :, Sk - 100:, :] = 1.0
    v[:, :, :50, 0] = 2.0
    if path == "bf16":
        o, lse = attn.fwd(q, k, v, causal=0)
    else:
        ops = attn.mxfp8_quantize_rows(q) + attn.mxfp8_quantize_rows(k) + attn.mxfp8_quantize_vt(v)
        del k, v
        o, lse = attn.fwd_fp8(*ops, causal=0)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert ("split" in attn.last_dispatch()) == (Sq == 1)
    ref = np.full((B, Hq, Sq, d), 100.0 / Sk)
    ref[..., 0] = 200.0 / Sk
    assert np.abs(o - ref).max() <= 2.0 ** -8 * ref.max(), (o[0, 0, 0, :4], ref[0, 0, 0, :4])
    assert np.abs(lse - np.log(Sk)).max() <= 1e-3
