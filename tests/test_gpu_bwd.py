"""Backward parity on the GPU: dQ, dK, dV from the HIP path against the
FP64 oracle's analytic gradients on the same seeded inputs."""
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


def _fwd_bwd(attn, w, fused=False):
    import torch
    x = synth.make_inputs(w, backward=True)
    dev = {n: to_device(x[n], w.dtype) for n in ("q", "k", "v", "do")}
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
    dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=w.causal, scale=w.scale,
                          fused=fused)
    torch.cuda.synchronize()
    out = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    return x, dev, out


SMALL = [
    # B, Hq, Hkv, Sq, Sk, d, causal
    (1, 2, 2, 200, 200, 64, 0),
    (1, 2, 2, 200, 200, 128, 1),
    (1, 4, 2, 190, 300, 128, 2),
    (2, 4, 1, 300, 170, 64, 1),
    (1, 2, 2, 150, 60, 128, 2),     # Sq > Sk bottom-right: fully masked query rows
    (1, 8, 2, 64, 64, 128, 0),      # one tile each way
    (1, 3, 1, 1, 77, 64, 0),        # a single query row
    (1, 2, 1, 130, 250, 64, 2),     # d = 64, bottom-right, 2 query heads per KV head
    (1, 8, 2, 520, 520, 128, 1),    # 17 query tiles x 4 query heads per KV head: unrolled loops, head changes
    (1, 4, 4, 96, 1000, 64, 0),     # Sk >> Sq, no mask: eight 128-key workgroups per head
]


@pytest.mark.parametrize("fused", [False, True], ids=["two_pass", "fused"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small_all_outputs(attn, shape, fused):
    B, Hq, Hkv, Sq, Sk, d, causal = shape
    w = synth.Workload("small_bwd", B, Hq, Hkv, Sq, Sk, d, "bf16", causal, seed=2000 + sum(shape),
                       backward=True)
    _say("case", shape, "fused" if fused else "two-pass")
    x, dev, out = _fwd_bwd(attn, w, fused)
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v", "do")}
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal=causal, scale=w.scale)
    check_o(to_host_f64(out["o"]), o_ref, "bf16")
    check_lse(out["lse"].cpu().numpy().astype(np.float64), lse_ref)
    g = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal=causal, scale=w.scale)
    for n in ("dq", "dk", "dv"):
        r = check_grad(n, to_host_f64(out[n]), g[n])
        _say(f"  {n} rel fro {r:.3e}")
    disp = attn.last_dispatch()
    assert "bwd_dkdv" in disp and (("bwd_dq<" in disp) != fused) and (("fused dQ" in disp) == fused)


@pytest.mark.parametrize("fused", [False, True], ids=["two_pass", "fused"])
def test_masked_positions_get_exactly_zero_gradient(attn, fused):
    # top-left with Sk > Sq: keys >= Sq are seen by no query -> dK = dV = 0 exactly
    w = synth.Workload("zero_keys", 1, 4, 2, 100, 230, 128, "bf16", 1, seed=31, backward=True)
    x, dev, out = _fwd_bwd(attn, w, fused)
    dk = to_host_f64(out["dk"])
    dv = to_host_f64(out["dv"])
    assert (dk[:, :, 100:] == 0).all() and (dv[:, :, 100:] == 0).all()
    assert np.abs(dk[:, :, :100]).max() > 0
    # bottom-right with Sq > Sk: query rows i < Sq - Sk see no key -> dQ = 0 exactly
    w = synth.Workload("zero_rows", 1, 4, 4, 200, 90, 64, "bf16", 2, seed=32, backward=True)
    x, dev, out = _fwd_bwd(attn, w, fused)
    dq = to_host_f64(out["dq"])
    assert (dq[:, :, :110] == 0).all() and np.abs(dq[:, :, 110:]).max() > 0
    # no key at all: dQ = 0 (the fused path's sums stay at the zeros the first pass wrote)
    import torch
    q = dev["q"]
    kv = torch.empty(1, 4, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = attn.fwd(q, kv, kv, causal=0)
    dq0, _, _ = attn.bwd(q, kv, kv, o, lse, dev["do"], causal=0, fused=fused)
    torch.cuda.synchronize()
    assert (dq0.float() == 0).all()


def test_train_workload_full_size(attn):
    """Full-size forward + backward (B=1, H=32, S=8192, d=128, causal): every
    one of the 32 heads against the FP64 oracle, O, lse, dQ, dK and dV, with
    the relative Frobenius errors printed per head and over whole tensors."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    w = synth.get_workload("train_causal_d128")
    _say("workload", w.name)
    x, dev, out = _fwd_bwd(attn, w)
    for n in ("o", "dq", "dk", "dv"):
        assert torch.isfinite(out[n].float()).all(), n
    got = {n: to_host_f64(out[n]) for n in ("o", "dq", "dk", "dv")}
    lse = out["lse"].cpu().numpy().astype(np.float64)
    del dev, out
    assert w.Hq == w.Hkv == 32 and w.B == 1

    def one_head(h):
        f = {n: synth.to_f64(x[n][:, h:h + 1], "bf16") for n in ("q", "k", "v", "do")}
        o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal=w.causal, scale=w.scale)
        g = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal=w.causal, scale=w.scale)
        return h, o_ref, lse_ref, g

    sq = {n: 0.0 for n in ("dq", "dk", "dv")}       # squared error and reference norms, all heads
    ref = {n: 0.0 for n in ("dq", "dk", "dv")}
    with ThreadPoolExecutor(max_workers=4) as ex:
        for h, o_ref, lse_ref, g in ex.map(one_head, range(w.Hq)):
            eo = check_o(got["o"][:, h:h + 1], o_ref, "bf16")
            el = check_lse(lse[:, h:h + 1], lse_ref)
            rs = []
            for n in ("dq", "dk", "dv"):
                part = got[n][:, h:h + 1]
                rs.append(check_grad(f"{n}[head {h}]", part, g[n]))
                sq[n] += float(np.sum((part - g[n]) ** 2))
                ref[n] += float(np.sum(g[n] ** 2))
            _say(f"  head {h:2d}: O max err {eo:.2e}, lse max err {el:.2e}, rel fro dq {rs[0]:.3e} "
                 f"dk {rs[1]:.3e} dv {rs[2]:.3e}")
    for n in ("dq", "dk", "dv"):
        r = (sq[n] / ref[n]) ** 0.5
        _say(f"  all heads: {n} rel fro {r:.3e}")
        assert r <= 3e-2, f"{n}: whole-tensor relative Frobenius error {r:.3e}"


def test_backward_is_deterministic(attn):
    """The two-pass backward gives the same bits every run. The fused one gives
    the same dK and dV bits every run (no atomics there); its dQ is summed
    atomically in a varying order, and all three agree with the two-pass
    results to rounding."""
    import torch
    w = synth.Workload("det_bwd", 1, 4, 2, 300, 300, 128, "bf16", 1, seed=33, backward=True)
    x, dev, out = _fwd_bwd(attn, w)
    for _ in range(3):
        dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], dev["do"], causal=1)
        torch.cuda.synchronize()
        assert torch.equal(dq, out["dq"]) and torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])
    fq, fk, fv = attn.bwd(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], dev["do"], causal=1, fused=True)
    gq, gk, gv = attn.bwd(dev["q"], dev["k"], dev["v"], out["o"], out["lse"], dev["do"], causal=1, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(fk, gk) and torch.equal(fv, gv)
    # the same float32 terms summed in another order, then rounded to bf16
    for x, y in ((fq, out["dq"]), (fk, out["dk"]), (fv, out["dv"])):
        a, b = x.float(), y.float()
        assert torch.linalg.norm(a - b) <= 1e-2 * torch.linalg.norm(b)
        assert (a - b).abs().max() <= 1e-2 * b.abs().max()
