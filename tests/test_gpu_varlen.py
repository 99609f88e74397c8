"""Packed variable-length batches on the GPU: the HIP path through
attn_fwd_varlen / attn_bwd_varlen against the FP64 oracle's varlen functions
on the same seeded packed inputs, plus bit-equality with the dense entry
points where the two describe the same problem."""
import sys

import numpy as np
import pytest

import oracle
import synth
from parity import check_grad, check_lse, check_o, to_device, to_host_f64

pytestmark = pytest.mark.gpu


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


def _w(name, Hq, Hkv, d, dtype, causal, lq, lk, seed, backward=False):
    return synth.VarlenWorkload(name, Hq, Hkv, d, dtype, causal, seed=seed, lens_q=tuple(lq),
                                lens_k=tuple(lk), backward=backward)


def _inputs(w):
    x = synth.make_varlen_inputs(w)
    dev = {n: to_device(x[n], w.dtype) for n in ("q", "k", "v") + (("do",) if w.backward else ())}
    f = {n: synth.to_f64(x[n], w.dtype) for n in ("q", "k", "v") + (("do",) if w.backward else ())}
    return x, dev, f


FWD_CASES = [
    # name, Hq, Hkv, d, dtype, causal, query lengths, key lengths
    ("mixed_causal", 8, 2, 128, "bf16", 1, (300, 0, 77, 1, 512), (300, 0, 77, 1, 512)),
    ("bottom_right", 4, 1, 64, "bf16", 2, (150, 40, 1, 250), (60, 300, 900, 250)),
    ("no_keys_f32", 2, 2, 64, "f32", 0, (33, 200, 0, 5), (10, 0, 5, 64)),
    ("decode_rows", 32, 8, 128, "bf16", 0, (1, 1, 1, 1), (4096, 100, 7000, 1)),
    ("tiny_tail", 2, 2, 128, "bf16", 1, (1, 2, 3, 129, 64), (1, 2, 3, 129, 64)),
    ("f32_causal", 4, 2, 128, "f32", 2, (100, 17), (120, 3)),
    # eight head units: each XCD takes one head of every sequence
    ("per_xcd_heads", 8, 8, 128, "bf16", 1, (200, 0, 1, 333, 64), (200, 9, 1, 333, 64)),
    # decode-shaped sequences (split over the keys) next to packed prefill ones
    ("decode_and_prefill", 8, 2, 128, "bf16", 0, (1, 300, 2, 77), (500, 300, 1000, 77)),
    # more sequences than one packed launch takes
    ("many_sequences", 4, 4, 64, "bf16", 1,
     tuple(int(x) for x in np.random.default_rng(71).integers(0, 90, 70)),
     tuple(int(x) for x in np.random.default_rng(71).integers(0, 90, 70))),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: c[0])
def test_fwd_varlen_matches_oracle(attn, case):
    import torch
    name, Hq, Hkv, d, dtype, causal, lq, lk = case
    w = _w(name, Hq, Hkv, d, dtype, causal, lq, lk, seed=3000 + len(name))
    _say(f"[fwd_varlen] {name} lens_q={lq} lens_k={lk}")
    x, dev, f = _inputs(w)
    o, lse = attn.fwd_varlen(dev["q"], dev["k"], dev["v"], x["cu_seqlens_q"], x["cu_seqlens_k"],
                             causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert attn.last_dispatch().startswith(f"attn_fwd_varlen: {sum(1 for n in lq if n)} sequences")
    o_ref, lse_ref = oracle.attention_forward_varlen(f["q"], f["k"], f["v"], x["cu_seqlens_q"],
                                                     x["cu_seqlens_k"], causal=causal, scale=w.scale)
    check_o(to_host_f64(o), o_ref, dtype)
    check_lse(to_host_f64(lse), lse_ref, tol=1e-5 if dtype == "f32" else 1e-3)


def test_fwd_varlen_writes_every_query_row(attn):
    # outputs start as garbage; sequences without queries (one of them with
    # keys) sit on both sides of the only one that has rows
    import torch
    w = _w("untouched", 2, 2, 64, "bf16", 1, (0, 70, 0), (40, 70, 9), seed=3100)
    x, dev, f = _inputs(w)
    o = torch.full_like(dev["q"], 7.0)
    lse = torch.full((2, 70), 7.0, device="cuda")
    attn.fwd_varlen(dev["q"], dev["k"], dev["v"], x["cu_seqlens_q"], x["cu_seqlens_k"], causal=1,
                    out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_varlen(f["q"], f["k"], f["v"], x["cu_seqlens_q"],
                                                     x["cu_seqlens_k"], causal=1, scale=w.scale)
    check_o(to_host_f64(o), o_ref, "bf16")
    check_lse(to_host_f64(lse), lse_ref)


@pytest.mark.parametrize("dtype,causal", [("bf16", 1), ("bf16", 2), ("f32", 0)])
def test_fwd_varlen_equal_lengths_bit_equal_to_dense(attn, dtype, causal):
    # the same kernels on the same rows: the packed call must give the same bits
    import torch
    B, Hq, Hkv, Sq, Sk, d = 3, 8, 2, 200, 260, 128
    wd = synth.Workload("dense_vs_packed", B, Hq, Hkv, Sq, Sk, d, dtype, causal, seed=3200 + causal)
    x = synth.make_inputs(wd)
    dev = {n: to_device(x[n], dtype) for n in ("q", "k", "v")}
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], causal=causal)
    pack = lambda t: t.transpose(0, 1).contiguous().reshape(t.shape[1], -1, d)
    cq, ck = synth.cu_seqlens([Sq] * B), synth.cu_seqlens([Sk] * B)
    ov, lv = attn.fwd_varlen(pack(dev["q"]), pack(dev["k"]), pack(dev["v"]), cq, ck, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(ov, pack(o))
    assert torch.equal(lv, lse.transpose(0, 1).reshape(Hq, -1))


BWD_CASES = [
    ("mixed_causal", 8, 2, 128, 1, (200, 0, 130, 64), (200, 50, 250, 64)),
    ("bottom_right", 4, 4, 64, 2, (150, 33, 1), (60, 200, 77)),
    ("no_mask_gqa", 4, 1, 128, 0, (96, 300), (500, 31)),
    ("no_queries_no_keys", 2, 2, 64, 1, (0, 90, 40), (70, 90, 0)),
    ("per_xcd_heads", 8, 8, 128, 2, (260, 0, 31, 1), (200, 64, 31, 700)),
    ("many_sequences", 2, 1, 64, 1,
     tuple(int(x) for x in np.random.default_rng(72).integers(0, 70, 67)),
     tuple(int(x) for x in np.random.default_rng(73).integers(0, 70, 67))),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: c[0])
def test_bwd_varlen_matches_oracle(attn, case):
    import torch
    name, Hq, Hkv, d, causal, lq, lk = case
    w = _w(name, Hq, Hkv, d, "bf16", causal, lq, lk, seed=3300 + len(name), backward=True)
    _say(f"[bwd_varlen] {name} lens_q={lq} lens_k={lk}")
    x, dev, f = _inputs(w)
    cq, ck = x["cu_seqlens_q"], x["cu_seqlens_k"]
    o, lse = attn.fwd_varlen(dev["q"], dev["k"], dev["v"], cq, ck, causal=causal)
    # dk/dv start as garbage: rows of a sequence without queries must come back as zeros
    dk = torch.full_like(dev["k"], 3.0)
    dv = torch.full_like(dev["v"], 3.0)
    dq, dk, dv = attn.bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cq, ck, causal=causal,
                                 dk=dk, dv=dv)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_forward_varlen(f["q"], f["k"], f["v"], cq, ck, causal=causal,
                                                     scale=w.scale)
    check_o(to_host_f64(o), o_ref, "bf16")
    check_lse(to_host_f64(lse), lse_ref)
    g = oracle.attention_backward_varlen(f["q"], f["k"], f["v"], f["do"], cq, ck, causal=causal,
                                         scale=w.scale)
    got = {"dq": to_host_f64(dq), "dk": to_host_f64(dk), "dv": to_host_f64(dv)}
    for n in ("dq", "dk", "dv"):
        check_grad(n, got[n], g[n])
    for b in range(len(lq)):
        if lq[b] == 0:       # keys nobody queries: exactly zero gradient
            assert (got["dk"][:, ck[b]:ck[b + 1]] == 0).all() and (got["dv"][:, ck[b]:ck[b + 1]] == 0).all()
        if lk[b] == 0:       # queries with no key: exactly zero dq
            assert (got["dq"][:, cq[b]:cq[b + 1]] == 0).all()


def test_bwd_varlen_equal_lengths_bit_equal_to_dense(attn):
    import torch
    B, Hq, Hkv, S, d = 2, 8, 2, 300, 128
    wd = synth.Workload("dense_vs_packed_bwd", B, Hq, Hkv, S, S, d, "bf16", 1, seed=3400, backward=True)
    x = synth.make_inputs(wd, backward=True)
    dev = {n: to_device(x[n], "bf16") for n in ("q", "k", "v", "do")}
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], causal=1)
    dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=1)
    pack = lambda t: t.transpose(0, 1).contiguous().reshape(t.shape[1], -1, d)
    cu = synth.cu_seqlens([S] * B)
    lse_p = lse.transpose(0, 1).contiguous().reshape(Hq, -1)
    g = attn.bwd_varlen(pack(dev["q"]), pack(dev["k"]), pack(dev["v"]), pack(o), lse_p, pack(dev["do"]),
                        cu, cu, causal=1)
    torch.cuda.synchronize()
    for a, b in zip(g, (dq, dk, dv)):
        assert torch.equal(a, pack(b))


def test_varlen_mix_full_size_sampled(attn):
    """The packed workload the benchmark times, at its full size, in the same
    launch configuration: every output is finite, and sampled query rows of
    sampled sequences match the oracle computed row by row; the backward is
    checked on whole heads of the shortest and the longest sequence."""
    import torch
    w = synth.VARLEN_WORKLOADS["varlen_mix_causal_d128"]
    lq, lk = synth.varlen_lengths(w)
    _say(f"[varlen full] {w.name} B={len(lq)} total={sum(lq)}")
    x, dev, f = _inputs(w)
    cq, ck = x["cu_seqlens_q"], x["cu_seqlens_k"]
    o, lse = attn.fwd_varlen(dev["q"], dev["k"], dev["v"], cq, ck, causal=w.causal)
    dq, dk, dv = attn.bwd_varlen(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], cq, ck, causal=w.causal)
    torch.cuda.synchronize()
    oh, lh = to_host_f64(o), to_host_f64(lse)
    assert np.isfinite(oh).all() and np.isfinite(lh).all()
    rng = np.random.default_rng(5)
    for b in rng.choice(len(lq), size=4, replace=False):
        S = lq[b]
        rows = np.unique(np.concatenate([[0, S - 1], rng.choice(S, size=6, replace=False)]))
        for h in rng.choice(w.Hq, size=2, replace=False):
            qs = f["q"][None, h:h + 1, cq[b] + rows]
            ks = f["k"][None, h:h + 1, ck[b]:ck[b + 1]]
            vs = f["v"][None, h:h + 1, ck[b]:ck[b + 1]]
            o_ref, l_ref = oracle.attention_forward(qs, ks, vs, causal=w.causal, scale=w.scale, rows=rows, Sq=S)
            check_o(oh[h, cq[b] + rows], o_ref[0, 0], "bf16")
            check_lse(lh[h, cq[b] + rows], l_ref[0, 0])
    got = {"dq": to_host_f64(dq), "dk": to_host_f64(dk), "dv": to_host_f64(dv)}
    for n in got:
        assert np.isfinite(got[n]).all(), n
    for b in (int(np.argmin(lq)), int(np.argmax(lq))):
        qs, ks = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        for h in (0, w.Hq - 1):
            g = oracle.attention_backward(f["q"][None, h:h + 1, qs], f["k"][None, h:h + 1, ks],
                                          f["v"][None, h:h + 1, ks], f["do"][None, h:h + 1, qs],
                                          causal=w.causal, scale=w.scale)
            check_grad("dq", got["dq"][h, qs], g["dq"][0, 0])
            check_grad("dk", got["dk"][h, ks], g["dk"][0, 0])
            check_grad("dv", got["dv"][h, ks], g["dv"][0, 0])
