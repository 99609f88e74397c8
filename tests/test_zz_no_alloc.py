"""attn_fwd_noalloc (static scratch, no allocation) against attn_fwd on the
GPU: two decode calls in a row, the second smaller, each bit-equal to the
workspace path and within the bf16 tolerances of the FP64 oracle; then a
prefill-shaped call, which needs no scratch."""
import sys

import numpy as np
import pytest

import oracle
import synth
from parity import check_lse, check_o, to_device, to_host_f64

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


def _case(attn, w):
    import torch
    x = synth.make_inputs(w)
    dev = {n: to_device(x[n], w.dtype) for n in ("q", "k", "v")}
    o_ref_dev, lse_ref_dev = attn.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale)
    o = torch.empty_like(dev["q"])
    lse = torch.empty(w.B, w.Hq, w.Sq, dtype=torch.float32, device="cuda")
    attn.fwd_noalloc(dev["q"], dev["k"], dev["v"], o, lse, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    disp = attn.last_dispatch()
    return x, o, lse, o_ref_dev, lse_ref_dev, disp


def _check_against_oracle(x, w, o, lse):
    f = {n: synth.to_f64(x[n], w.dtype) for n in ("q", "k", "v")}
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal=w.causal, scale=w.scale)
    check_o(to_host_f64(o), o_ref, "bf16")
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref)


def test_noalloc_two_calls_then_prefill(attn):
    import torch
    # 1: the grouped-query decode (16 x 32 query rows, 32768 keys): 4 MiB of partials
    big = synth.get_workload("gqa_decode")
    # 2: a smaller decode on the same scratch, whose first bytes still hold call 1's partials
    small = synth.Workload("noalloc_small", 2, 8, 2, 1, 1000, 128, "bf16", 0, seed=91)
    for w in (big, small):
        _say("case", w.name, (w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d))
        assert 0 < attn.fwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, w.causal,
                                            attn.ATTN_BF16) <= attn.NOALLOC_SCRATCH_BYTES
        x, o, lse, o_ws, lse_ws, disp = _case(attn, w)
        assert "static scratch" in disp and "fwd_split_bf16" in disp, disp
        assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws), "differs from attn_fwd with a workspace"
        _check_against_oracle(x, w, o, lse)
    # 3: prefill-shaped (no scratch used)
    w = synth.Workload("noalloc_prefill", 1, 4, 2, 200, 260, 64, "bf16", 1, seed=92)
    _say("case", w.name)
    x, o, lse, o_ws, lse_ws, disp = _case(attn, w)
    assert "static scratch" not in disp and "fwd_prefill" in disp, disp
    assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
    _check_against_oracle(x, w, o, lse)
