"""Helpers for the GPU parity tests: host<->device marshalling of the seeded
inputs and the tolerance checks (not a test module)."""
from __future__ import annotations

import numpy as np

import synth

# Tolerances of the library, checked after a finiteness check.
F32_MAX_ABS = 1e-5
BF16_ABS = 2e-2
BF16_REL = 2e-2
LSE_ABS = 1e-3
GRAD_REL_FRO = 3e-2


def to_device(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16))
        return t.cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_host_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.f32_from_bf16_bits(bits).astype(np.float64)
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_finite(name: str, x: np.ndarray, allow_neg_inf: bool = False):
    bad = np.isnan(x) | np.isposinf(x)
    if not allow_neg_inf:
        bad |= np.isneginf(x)
    assert not bad.any(), f"{name}: {int(bad.sum())} non-finite values"


def check_o(o: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = "O"):
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert_finite(what, o)
    err = np.abs(o - o_ref)
    if dtype == "f32":
        worst = err.max() if err.size else 0.0
        assert worst <= F32_MAX_ABS, f"{what}: max abs err {worst:.3e} > {F32_MAX_ABS}"
        return worst
    bound = BF16_ABS + BF16_REL * np.abs(o_ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside 2e-2 + 2e-2|ref|; "
                           f"worst err {err.max():.3e}")
    return err.max() if err.size else 0.0


def check_lse(lse: np.ndarray, lse_ref: np.ndarray, tol: float = LSE_ABS):
    assert lse.shape == lse_ref.shape
    assert not np.isnan(lse).any() and not np.isposinf(lse).any()
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf), "lse = -inf exactly where no key is visible"
    fin = ~ninf
    if fin.any():
        worst = np.abs(lse[fin] - lse_ref[fin]).max()
        assert worst <= tol, f"lse: max abs err {worst:.3e} > {tol}"
        return worst
    return 0.0


def rel_fro(g: np.ndarray, g_ref: np.ndarray) -> float:
    den = np.linalg.norm(g_ref)
    num = np.linalg.norm(g - g_ref)
    return float(num / den) if den > 0 else float(num)


def check_grad(name: str, g: np.ndarray, g_ref: np.ndarray, per_head_axis: int = 1):
    assert g.shape == g_ref.shape
    assert_finite(name, g)
    r = rel_fro(g, g_ref)
    assert r <= GRAD_REL_FRO, f"{name}: relative Frobenius error {r:.3e} > {GRAD_REL_FRO}"
    return r
