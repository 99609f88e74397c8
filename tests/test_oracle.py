"""Pins for the FP64 oracle: values printed on the pages, closed forms,
library routines, brute force and central differences (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (FullyMaskedRowError, attention_backward, attention_backward_varlen,
                    attention_forward, attention_forward_varlen, dropout_keep_mask,
                    dropout_threshold, merge_states, online_softmax_forward, philox4x32_10,
                    visible_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _rand(rng, B, Hq, Hkv, Sq, Sk, d, dv=None, outliers=0, factor=30.0):
    dv = d if dv is None else dv
    q = rng.standard_normal((B, Hq, Sq, d))
    k = rng.standard_normal((B, Hkv, Sk, d))
    v = rng.standard_normal((B, Hkv, Sk, dv))
    if outliers:
        for b in range(B):
            for h in range(Hq):
                rows = rng.choice(Sq, size=outliers, replace=False)
                q[b, h, rows] *= factor
    return q, k, v


# ---------------------------------------------------------------- worked example
def _worked_inputs(g):
    q = np.ones((1, 1, 1, 1))
    k = np.array(g["scores"], dtype=np.float64).reshape(1, 1, 3, 1)
    v = np.array(g["values"], dtype=np.float64).reshape(1, 1, 3, 1)
    return q, k, v


def test_worked_example_states_and_output():
    g = _load("worked_example.json")
    q, k, v = _worked_inputs(g)
    tol = 0.5 * 10 ** (-g["printed_decimals"])
    o, lse, states = online_softmax_forward(q, k, v, tile=g["tile"], scale=1.0, trace=True)
    assert len(states) == 3
    for (m, l, u), (m_p, l_p, u_p) in zip(states, g["states_m_l_u"]):
        assert abs(m[0] - m_p) <= tol and abs(l[0] - l_p) <= tol and abs(u[0, 0] - u_p) <= tol
    assert abs(o.item() - g["output"]) <= tol
    o2, lse2 = attention_forward(q, k, v, scale=1.0)
    assert abs(o2.item() - g["output"]) <= tol
    # lse closed form: 1001 + ln(1 + e^-1 + e^-2)
    expect = 1001.0 + math.log(1.0 + math.exp(-1.0) + math.exp(-2.0))
    assert abs(lse.item() - expect) < 1e-12 and abs(lse2.item() - expect) < 1e-12


def test_worked_example_direct_exp_overflows_but_oracle_is_finite():
    g = _load("worked_example.json")
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float64(g["scores"][1])))   # e^1001 > DBL_MAX
    q, k, v = _worked_inputs(g)
    o, lse = attention_forward(q, k, v, scale=1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


# ---------------------------------------------------------------- tile invariance
@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("tile", [1, 2, 3, 8, 16, 37, 1000])
def test_tile_invariance(causal, tile):
    g = _load("tile_invariance.json")
    assert g["printed_max_abs_error"] == [0.0] * 4
    rng = np.random.default_rng(100 + causal)
    Sq, Sk = (45, 45) if causal != 2 else (37, 53)
    q, k, v = _rand(rng, 1, 2, 1, Sq, Sk, 8, outliers=3)
    o_ref, lse_ref = attention_forward(q, k, v, causal=causal)
    o, lse = online_softmax_forward(q, k, v, tile=tile, causal=causal)
    assert np.abs(o - o_ref).max() <= 1e-12
    assert np.abs(lse - lse_ref).max() <= 1e-12 * max(1.0, np.abs(lse_ref).max())


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("causal", [1, 2])
def test_single_visible_key(causal):
    rng = np.random.default_rng(7)
    Sq, Sk = (9, 9) if causal == 1 else (9, 5)
    q, k, v = _rand(rng, 1, 1, 1, Sq, Sk, 4)
    o, lse = attention_forward(q, k, v, causal=causal, scale=0.7)
    row = 0 if causal == 1 else Sq - Sk        # first row that sees exactly key 0
    assert np.array_equal(o[0, 0, row], v[0, 0, 0])
    assert lse[0, 0, row] == pytest.approx(0.7 * q[0, 0, row] @ k[0, 0, 0], abs=1e-14)


def test_uniform_values():
    rng = np.random.default_rng(8)
    q, k, _ = _rand(rng, 2, 2, 2, 6, 11, 4)
    vrow = rng.standard_normal(4)
    v = np.broadcast_to(vrow, (2, 2, 11, 4)).copy()
    for causal in (0, 1):
        o, _ = attention_forward(q, k, v, causal=causal)
        assert np.abs(o - vrow).max() < 1e-14


@pytest.mark.parametrize("causal", [0, 1, 2])
def test_zero_keys_give_mean_of_visible_values(causal):
    rng = np.random.default_rng(9)
    Sq, Sk = 7, 10
    q, _, v = _rand(rng, 1, 1, 1, Sq, Sk, 3)
    k = np.zeros((1, 1, Sk, 3))
    o, lse = attention_forward(q, k, v, causal=causal)
    vis = visible_mask(Sq, Sk, causal)
    for i in range(Sq):
        n = vis[i].sum()
        assert np.allclose(o[0, 0, i], v[0, 0, vis[i]].mean(axis=0), atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)


# ---------------------------------------------------------------- invariants
def test_bounds_and_lse_range():
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 1, 3, 3, 20, 33, 8, outliers=2)
    for causal in (0, 1, 2):
        o, lse = attention_forward(q, k, v, causal=causal)
        vis = visible_mask(20, 33, causal)
        s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(8)
        for h in range(3):
            for i in range(20):
                vv = v[0, h, vis[i]]
                assert (o[0, h, i] >= vv.min(axis=0) - 1e-12).all()
                assert (o[0, h, i] <= vv.max(axis=0) + 1e-12).all()
                smax = s[0, h, i, vis[i]].max()
                assert smax - 1e-12 <= lse[0, h, i] <= smax + math.log(vis[i].sum()) + 1e-12


def test_key_shift_and_permutation():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 1, 2, 2, 12, 17, 5)
    w = rng.standard_normal(5)
    o, lse = attention_forward(q, k, v, causal=0, scale=0.4)
    o2, lse2 = attention_forward(q, k + w, v, causal=0, scale=0.4)
    assert np.abs(o2 - o).max() < 1e-12
    assert np.abs(lse2 - (lse + 0.4 * (q @ w))).max() < 1e-12
    perm = rng.permutation(17)
    o3, lse3 = attention_forward(q, k[:, :, perm], v[:, :, perm], causal=0, scale=0.4)
    assert np.abs(o3 - o).max() < 1e-12 and np.abs(lse3 - lse).max() < 1e-12


def test_rows_subset_matches_full():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 2, 4, 2, 30, 41, 6)
    rows = np.array([0, 3, 17, 29])
    for causal in (0, 1, 2):
        o, lse = attention_forward(q, k, v, causal=causal)
        os_, lses = attention_forward(q[:, :, rows], k, v, causal=causal, rows=rows, Sq=30)
        assert np.array_equal(os_, o[:, :, rows]) and np.array_equal(lses, lse[:, :, rows])


# ---------------------------------------------------------------- library routines
def _torch_mask(Sq, Sk, causal):
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Sk)[None, :]
    if causal == 0:
        return torch.ones(Sq, Sk, dtype=torch.bool)
    if causal == 1:
        return j <= i
    return j <= i + (Sk - Sq)


@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("gqa", [False, True])
def test_forward_matches_torch_sdpa_fp64(causal, gqa):
    rng = np.random.default_rng(13)
    Hq, Hkv = (4, 2) if gqa else (3, 3)
    Sq, Sk = (19, 19) if causal == 1 else (13, 29)
    q, k, v = _rand(rng, 2, Hq, Hkv, Sq, Sk, 8, dv=8, outliers=2)
    o, lse = attention_forward(q, k, v, causal=causal, scale=0.3)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    if causal == 1:
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.3,
                                                               enable_gqa=gqa)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=_torch_mask(Sq, Sk, causal), scale=0.3, enable_gqa=gqa)
    assert np.abs(o - ref.numpy()).max() < 1e-12
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    s = 0.3 * tq @ kk.transpose(-1, -2)
    s = s.masked_fill(~_torch_mask(Sq, Sk, causal), float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, dim=-1).numpy()).max() < 1e-12


def test_forward_matches_literal_softmax_brute_force():
    # exp(s_j) / sum_k exp(s_k) with no max subtraction, scores kept small
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 1, 1, 1, 4, 6, 3)
    o, lse = attention_forward(q, k, v, causal=2, scale=0.5)
    for i in range(4):
        keys = [j for j in range(6) if j <= i + 2]
        e = {j: math.exp(0.5 * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(3))) for j in keys}
        z = sum(e.values())
        for c in range(3):
            assert o[0, 0, i, c] == pytest.approx(sum(e[j] * v[0, 0, j, c] for j in keys) / z, abs=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(z), abs=1e-14)


# ---------------------------------------------------------------- fully masked rows
def test_fully_masked_rows_strict_and_defined():
    rng = np.random.default_rng(15)
    Sq, Sk = 9, 4                      # causal=2: rows 0..4 see no key
    q, k, v = _rand(rng, 1, 2, 1, Sq, Sk, 4)
    with pytest.raises(FullyMaskedRowError):
        attention_forward(q, k, v, causal=2, strict=True)
    o, lse = attention_forward(q, k, v, causal=2)
    assert np.isfinite(o).all()
    assert (o[:, :, :5] == 0).all() and np.isneginf(lse[:, :, :5]).all()
    assert np.isfinite(lse[:, :, 5:]).all()
    for tile in (1, 3, 8):
        o2, lse2 = online_softmax_forward(q, k, v, tile=tile, causal=2)
        assert np.abs(o2 - o).max() < 1e-12
        assert np.array_equal(np.isneginf(lse2), np.isneginf(lse))
    g = attention_backward(q, k, v, rng.standard_normal(o.shape), causal=2)
    assert (g["dq"][:, :, :5] == 0).all()
    assert all(np.isfinite(g[n]).all() for n in ("dq", "dk", "dv"))
    # Sk = 0: every row empty
    o0, lse0 = attention_forward(q, k[:, :, :0], v[:, :, :0], causal=0)
    assert (o0 == 0).all() and np.isneginf(lse0).all()


def test_overflow_rows_stay_finite():
    rng = np.random.default_rng(16)
    q, k, v = _rand(rng, 1, 2, 2, 64, 64, 16, outliers=4, factor=300.0)
    o, lse = attention_forward(q, k, v, causal=1)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.abs(lse).max() > 709.8       # beyond ln(DBL_MAX): a direct exp would overflow
    o2, lse2 = online_softmax_forward(q, k, v, tile=5, causal=1)
    assert np.abs(o2 - o).max() < 1e-12


# ---------------------------------------------------------------- merge rule
def test_merge_states_equals_single_pass():
    rng = np.random.default_rng(17)
    q, k, v = _rand(rng, 2, 4, 2, 1, 50, 8)
    o, lse = attention_forward(q, k, v)
    cut = 19
    oa, la = attention_forward(q, k[:, :, :cut], v[:, :, :cut])
    ob, lb = attention_forward(q, k[:, :, cut:], v[:, :, cut:])
    om, lm = merge_states(oa, la, ob, lb)
    assert np.abs(om - o).max() < 1e-13 and np.abs(lm - lse).max() < 1e-13
    # an empty part weighs nothing
    oe, le = attention_forward(q, k[:, :, :0], v[:, :, :0])
    om2, lm2 = merge_states(o, lse, oe, le)
    assert np.abs(om2 - o).max() == 0 and np.abs(lm2 - lse).max() == 0


# ---------------------------------------------------------------- gradients
def _loss_half_sq(q, k, v, causal):
    o, _ = attention_forward(q, k, v, causal=causal)
    return 0.5 * float((o ** 2).sum()), o


def test_central_differences_masked_2x3x2():
    g = _load("gradient_check.json")
    rng = np.random.default_rng(18)
    q, k, v = _rand(rng, 1, 1, 1, 2, 3, 2)
    causal = 2                               # first query may not read the third key
    vis = visible_mask(2, 3, causal)
    assert vis.tolist() == [[True, True, False], [True, True, True]]
    _, o = _loss_half_sq(q, k, v, causal)
    grads = attention_backward(q, k, v, o, causal=causal, return_intermediates=True)
    h = 1e-6
    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            args_m = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num = (_loss_half_sq(*args_p, causal)[0] - _loss_half_sq(*args_m, causal)[0]) / (2 * h)
            worst = max(worst, abs(num - grads[name][idx]))
    assert worst <= 1e-8, worst
    assert g["printed_max_abs_error"] < 1e-8        # the page's own run is in the same regime
    ds = grads["ds"][0, 0]
    assert ds[0, 2] == 0.0                           # masked score: exactly zero gradient
    assert np.abs(ds.sum(axis=1)).max() <= 1e-14     # shift invariance of softmax


@pytest.mark.parametrize("causal", [0, 1, 2])
@pytest.mark.parametrize("shape", [(1, 2, 2, 7, 7, 4), (2, 4, 2, 5, 9, 8), (1, 4, 1, 9, 6, 3)])
def test_backward_matches_torch_autograd_fp64(causal, shape):
    B, Hq, Hkv, Sq, Sk, d = shape
    rng = np.random.default_rng(19 + causal)
    q, k, v = _rand(rng, B, Hq, Hkv, Sq, Sk, d, outliers=1)
    do = rng.standard_normal((B, Hq, Sq, d))
    gr = attention_backward(q, k, v, do, causal=causal, scale=0.45, return_intermediates=True)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    g = Hq // Hkv
    kk, vv = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
    s = 0.45 * tq @ kk.transpose(-1, -2)
    mask = _torch_mask(Sq, Sk, causal)
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)                 # fully masked rows (causal=2, Sq>Sk)
    o = p @ vv
    o.backward(torch.from_numpy(do))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.abs(gr[name] - t.grad.numpy()).max() < 1e-12, name
    # the Jacobian row term equals dO . O (the identity the GPU backward uses)
    o_np, _ = attention_forward(q, k, v, causal=causal, scale=0.45)
    assert np.abs(gr["D"] - (do * o_np).sum(-1)).max() < 1e-12
    assert np.abs(gr["ds"].sum(-1)).max() < 1e-12
    assert (gr["ds"][..., ~mask] == 0).all()


def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(20)
    q, k, v = _rand(rng, 1, 6, 2, 8, 8, 4)
    do = rng.standard_normal(q.shape)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o, lse = attention_forward(q, k, v, causal=1)
    o2, lse2 = attention_forward(q, kr, vr, causal=1)
    assert np.abs(o - o2).max() < 1e-14 and np.abs(lse - lse2).max() < 1e-14
    g1 = attention_backward(q, k, v, do, causal=1)
    g2 = attention_backward(q, kr, vr, do, causal=1)
    assert np.abs(g1["dq"] - g2["dq"]).max() < 1e-13
    assert np.abs(g1["dk"] - g2["dk"].reshape(1, 2, 3, 8, 4).sum(2)).max() < 1e-13
    assert np.abs(g1["dv"] - g2["dv"].reshape(1, 2, 3, 8, 4).sum(2)).max() < 1e-13


def test_keys_no_query_sees_get_zero_gradient():
    rng = np.random.default_rng(21)
    q, k, v = _rand(rng, 1, 2, 2, 5, 9, 4)          # causal=1: keys 5..8 are never visible
    gr = attention_backward(q, k, v, rng.standard_normal(q.shape), causal=1)
    assert (gr["dk"][:, :, 5:] == 0).all() and (gr["dv"][:, :, 5:] == 0).all()


# ---------------------------------------------------------------- packed variable-length batches
VARLEN_LENS = {   # (query lengths, key lengths) per causal mode; zero-length sequences included
    0: ((5, 0, 7, 3), (6, 4, 7, 2)),
    1: ((5, 0, 7, 3), (6, 4, 7, 2)),
    2: ((5, 0, 7, 3), (3, 4, 9, 2)),      # sequence 0 has query rows that see no key
}


def _cu(lens):
    return [0] + list(np.cumsum(lens))


def _packed(rng, Hq, Hkv, lq, lk, d):
    tq, tk = sum(lq), sum(lk)
    return (rng.standard_normal((Hq, tq, d)), rng.standard_normal((Hkv, tk, d)),
            rng.standard_normal((Hkv, tk, d)))


def _block_diagonal_mask(lq, lk, causal):
    """[total_q, total_k] visibility from packed row numbers: a row sees a key
    of its own sequence only, and the causal rule compares logical positions
    (packed number minus the sequence's first packed row)."""
    cq, ck = _cu(lq), _cu(lk)
    r = np.arange(cq[-1])
    c = np.arange(ck[-1])
    sr = np.searchsorted(cq, r, side="right") - 1        # sequence of each query row
    sc = np.searchsorted(ck, c, side="right") - 1        # sequence of each key row
    same = sr[:, None] == sc[None, :]
    i = (r - np.asarray(cq)[sr])[:, None]
    j = (c - np.asarray(ck)[sc])[None, :]
    Sq = np.asarray(lq)[sr][:, None]
    Sk = np.asarray(lk)[sr][:, None]
    if causal == 0:
        rule = np.ones_like(same)
    elif causal == 1:
        rule = j <= i
    else:
        rule = j <= i + (Sk - Sq)
    return same & rule


@pytest.mark.parametrize("causal", [0, 1, 2])
def test_varlen_matches_block_diagonal_softmax(causal):
    # one masked softmax over the whole packed matrix, by torch in fp64
    rng = np.random.default_rng(22 + causal)
    lq, lk = VARLEN_LENS[causal]
    q, k, v = _packed(rng, 4, 2, lq, lk, 6)
    o, lse = attention_forward_varlen(q, k, v, _cu(lq), _cu(lk), causal=causal, scale=0.4)
    mask = torch.from_numpy(_block_diagonal_mask(lq, lk, causal))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(2, dim=0), tv.repeat_interleave(2, dim=0)
    s = (0.4 * tq @ kk.transpose(-1, -2)).masked_fill(~mask, float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)
    assert np.abs(o - (p @ vv).numpy()).max() < 1e-12
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    assert np.array_equal(np.isinf(lse), np.isinf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12
    if causal == 2:
        assert np.isinf(lse[:, :2]).all() and (o[:, :2] == 0).all()   # 5 queries, 3 keys


def test_varlen_equal_lengths_equal_dense_batch():
    rng = np.random.default_rng(25)
    B, Hq, Hkv, Sq, Sk, d = 3, 4, 2, 6, 9, 5
    q, k, v = _rand(rng, B, Hq, Hkv, Sq, Sk, d)
    do = rng.standard_normal(q.shape)
    pack = lambda x: x.transpose(1, 0, 2, 3).reshape(x.shape[1], -1, x.shape[3])
    cq, ck = _cu([Sq] * B), _cu([Sk] * B)
    for causal in (0, 1, 2):
        o, lse = attention_forward(q, k, v, causal=causal)
        ov, lv = attention_forward_varlen(pack(q), pack(k), pack(v), cq, ck, causal=causal)
        assert np.abs(ov - pack(o)).max() < 1e-14
        assert np.abs(lv - lse.transpose(1, 0, 2).reshape(Hq, -1)).max() < 1e-14
        g = attention_backward(q, k, v, do, causal=causal)
        gv = attention_backward_varlen(pack(q), pack(k), pack(v), pack(do), cq, ck, causal=causal)
        for n in ("dq", "dk", "dv"):
            assert np.abs(gv[n] - pack(g[n])).max() < 1e-13, n


def test_varlen_empty_sequences():
    rng = np.random.default_rng(26)
    lq, lk = (3, 0, 2), (0, 4, 5)
    q, k, v = _packed(rng, 2, 1, lq, lk, 4)
    o, lse = attention_forward_varlen(q, k, v, _cu(lq), _cu(lk), causal=1)
    assert (o[:, :3] == 0).all() and np.isneginf(lse[:, :3]).all()      # no keys
    g = attention_backward_varlen(q, k, v, rng.standard_normal(q.shape), _cu(lq), _cu(lk), causal=1)
    assert (g["dq"][:, :3] == 0).all()
    assert (g["dk"][:, :4] == 0).all() and (g["dv"][:, :4] == 0).all()  # no queries
    assert np.abs(g["dk"][:, 4:]).max() > 0
    with pytest.raises(ValueError):
        attention_forward_varlen(q, k, v, [0, 3, 2, 5], _cu(lk))
    with pytest.raises(ValueError):
        attention_forward_varlen(q, k, v, [1, 3, 3, 5], _cu(lk))


def _varlen_loss(q, k, v, cq, ck, causal):
    o, _ = attention_forward_varlen(q, k, v, cq, ck, causal=causal, scale=0.7)
    return 0.5 * float((o ** 2).sum()), o


@pytest.mark.parametrize("causal", [1, 2])
def test_varlen_central_differences(causal):
    rng = np.random.default_rng(27 + causal)
    lq, lk = (2, 0, 3), (3, 2, 1)
    cq, ck = _cu(lq), _cu(lk)
    q, k, v = _packed(rng, 2, 1, lq, lk, 2)
    _, o = _varlen_loss(q, k, v, cq, ck, causal)
    gr = attention_backward_varlen(q, k, v, o, cq, ck, causal=causal, scale=0.7)
    h = 1e-6
    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            am = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num = (_varlen_loss(*ap, cq, ck, causal)[0] - _varlen_loss(*am, cq, ck, causal)[0]) / (2 * h)
            worst = max(worst, abs(num - gr[name][idx]))
    assert worst <= 1e-8, worst
    assert (gr["dk"][:, 3:5] == 0).all()                 # the keys of the sequence without queries


def test_varlen_backward_matches_autograd_block_diagonal():
    rng = np.random.default_rng(30)
    lq, lk = (4, 6, 1), (5, 6, 3)
    q, k, v = _packed(rng, 4, 2, lq, lk, 3)
    do = rng.standard_normal(q.shape)
    gr = attention_backward_varlen(q, k, v, do, _cu(lq), _cu(lk), causal=1, scale=0.5)
    mask = torch.from_numpy(_block_diagonal_mask(lq, lk, 1))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(2, dim=0), tv.repeat_interleave(2, dim=0)
    s = (0.5 * tq @ kk.transpose(-1, -2)).masked_fill(~mask, float("-inf"))
    (torch.softmax(s, dim=-1) @ vv).backward(torch.from_numpy(do))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.abs(gr[name] - t.grad.numpy()).max() < 1e-12, name


# ---------------------------------------------------------------- dropout
def test_philox_known_answer_vectors():
    for vec in _load("philox_kat.json")["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        out = philox4x32_10(np.array(ctr, dtype=np.uint64), key)
        assert ["%08x" % int(x) for x in out] == vec["output"]


def test_dropout_mask_layout_rate_and_streams():
    B, Hq, Sq, Sk, seed, off = 2, 3, 10, 13, (7 << 32) | 123, 5
    m = dropout_keep_mask(B, Hq, Sq, Sk, 0.3, seed, off)
    thr = dropout_threshold(0.3)
    assert thr == 77
    # element by element from single generator calls: counter (j//4, i//4, b*Hq+h, offset),
    # byte j%4 of word i%4
    for (b, h, i, j) in np.ndindex(m.shape):
        w = philox4x32_10(np.array([j // 4, i // 4, b * Hq + h, off], dtype=np.uint64), (123, 7))
        byte = (int(w[i % 4]) >> (8 * (j % 4))) & 0xFF
        assert m[b, h, i, j] == (byte >= thr), (b, h, i, j)
    big = dropout_keep_mask(1, 4, 256, 256, 0.1, 99, 0)
    keep = 1 - dropout_threshold(0.1) / 256
    n = big.size
    assert abs(big.mean() - keep) < 6 * np.sqrt(keep * (1 - keep) / n)
    assert dropout_keep_mask(1, 1, 8, 8, 0.0, 1, 0).all()
    assert not np.array_equal(big, dropout_keep_mask(1, 4, 256, 256, 0.1, 99, 1))
    assert np.array_equal(big, dropout_keep_mask(1, 4, 256, 256, 0.1, 99, 0))
    for bad in (-0.1, 1.0, 0.999, float("nan")):
        with pytest.raises(ValueError):
            dropout_threshold(bad)


def test_dropout_zero_probability_is_plain_attention():
    rng = np.random.default_rng(40)
    q, k, v = _rand(rng, 1, 4, 2, 9, 11, 4)
    do = rng.standard_normal(q.shape)
    o, lse = attention_forward(q, k, v, causal=2)
    o0, lse0 = attention_forward(q, k, v, causal=2, dropout=(0.0, 5, 0))
    assert np.array_equal(o, o0) and np.array_equal(lse, lse0)
    g = attention_backward(q, k, v, do, causal=2)
    g0 = attention_backward(q, k, v, do, causal=2, dropout=(0.0, 5, 0))
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(g[n], g0[n])


def _drop_loss(q, k, v, causal, drop):
    o, _ = attention_forward(q, k, v, causal=causal, scale=0.6, dropout=drop)
    return 0.5 * float((o ** 2).sum()), o


def test_dropout_central_differences():
    rng = np.random.default_rng(41)
    q, k, v = _rand(rng, 1, 2, 1, 5, 6, 3)
    drop = (0.4, 2024, 3)
    _, o = _drop_loss(q, k, v, 1, drop)
    gr = attention_backward(q, k, v, o, causal=1, scale=0.6, dropout=drop)
    h = 1e-6
    worst = 0.0
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = {"dq": (xp, k, v), "dk": (q, xp, v), "dv": (q, k, xp)}[name]
            am = {"dq": (xm, k, v), "dk": (q, xm, v), "dv": (q, k, xm)}[name]
            num = (_drop_loss(*ap, 1, drop)[0] - _drop_loss(*am, 1, drop)[0]) / (2 * h)
            worst = max(worst, abs(num - gr[name][idx]))
    assert worst <= 1e-8, worst


@pytest.mark.parametrize("causal", [0, 2])
def test_dropout_matches_torch_autograd_fp64(causal):
    rng = np.random.default_rng(42 + causal)
    B, Hq, Hkv, Sq, Sk, d = 2, 4, 2, 7, 10, 5
    q, k, v = _rand(rng, B, Hq, Hkv, Sq, Sk, d, outliers=1)
    do = rng.standard_normal((B, Hq, Sq, d))
    drop = (0.25, 77, 11)
    o, lse = attention_forward(q, k, v, causal=causal, scale=0.5, dropout=drop)
    gr = attention_backward(q, k, v, do, causal=causal, scale=0.5, dropout=drop)
    z = torch.from_numpy(dropout_keep_mask(B, Hq, Sq, Sk, *drop).astype(np.float64)) / (1 - 64 / 256)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    kk, vv = tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1)
    s = (0.5 * tq @ kk.transpose(-1, -2)).masked_fill(~_torch_mask(Sq, Sk, causal), float("-inf"))
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)
    ref = (p * z) @ vv
    assert np.abs(o - ref.detach().numpy()).max() < 1e-12
    assert np.abs(lse - torch.logsumexp(s, dim=-1).detach().numpy()).max() < 1e-12
    ref.backward(torch.from_numpy(do))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.abs(gr[name] - t.grad.numpy()).max() < 1e-12, name
