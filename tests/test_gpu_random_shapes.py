"""Forward and backward parity on seeded random shapes: batch, grouped-query
ratio, ragged query and key lengths (including single rows, lengths that are
not multiples of any tile and Sq > Sk with bottom-right alignment), d and the
three mask modes, each against the FP64 oracle with the same tolerances as
the fixed cases. The shapes come from a fixed seed, so every run checks the
same ones."""
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


def _shapes(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        causal = int(rng.integers(0, 3))
        # lengths: mostly ragged, sometimes a single row or a single key
        Sq = 1 if i % 7 == 3 else int(rng.integers(2, 600))
        Sk = 1 if i % 11 == 5 else int(rng.integers(2, 600))
        out.append((B, Hkv * g, Hkv, Sq, Sk, d, causal))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def attn():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_38_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("idx", range(len(SHAPES)), ids=lambda i: "x".join(map(str, SHAPES[i])))
def test_random_shape_fwd_bwd(attn, idx):
    import torch
    B, Hq, Hkv, Sq, Sk, d, causal = SHAPES[idx]
    fused = idx % 2 == 1
    _say("case", SHAPES[idx], "fused" if fused else "two-pass")
    w = synth.Workload("random_shape", B, Hq, Hkv, Sq, Sk, d, "bf16", causal, seed=5000 + idx, backward=True)
    x = synth.make_inputs(w, backward=True)
    dev = {n: to_device(x[n], w.dtype) for n in ("q", "k", "v", "do")}
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=w.scale)
    dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], causal=causal, scale=w.scale,
                          fused=fused)
    torch.cuda.synchronize()
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v", "do")}
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal=causal, scale=w.scale)
    check_o(to_host_f64(o), o_ref, "bf16")
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref)
    g = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal=causal, scale=w.scale)
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        r = check_grad(n, to_host_f64(t), g[n])
        _say(f"  {n} rel fro {r:.3e}")
