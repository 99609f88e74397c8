"""The seeded input generator: bf16 rounding against torch, determinism, recipe."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1, 30, 1e-3, 1e4)])
    # ties: values exactly halfway between two bf16 numbers
    base = synth.f32_from_bf16_bits(np.arange(0x3F80, 0x3F90, dtype=np.uint16)).view(np.uint32)
    ties = (base + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = synth.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.f32_from_bf16_bits(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_follow_recipe():
    w = synth.get_workload("single_head_f32")
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    for n in ("q", "k", "v"):
        assert np.array_equal(a[n], b[n]) and a[n].dtype == np.float32
    rng = np.random.Generator(np.random.PCG64(w.seed))
    assert np.array_equal(a["q"], rng.standard_normal((1, 1, 256, 64), dtype=np.float32))


def test_outlier_rows():
    w = synth.get_workload("long_causal_d128").with_(B=1, Hq=2, Hkv=2, Sq=300, Sk=300, d=16)
    x = synth.make_inputs(w)
    rows = x["outlier_rows"]
    assert rows.shape == (1, 2, 3)
    q = synth.to_f64(x["q"], "bf16")
    norms = np.linalg.norm(q, axis=-1)
    for h in range(2):
        assert len(set(rows[0, h].tolist())) == 3
        assert norms[0, h, rows[0, h]].min() > 10 * np.median(norms[0, h])


def test_oracle_and_library_do_not_import_each_other():
    import pathlib
    root = pathlib.Path(__file__).resolve().parent.parent
    for f in (root / "oracle").glob("*.py"):
        t = f.read_text()
        assert "exact_io_aware_38_amd" not in t and "import synth" not in t
    for f in (root / "exact_io_aware_38_amd").rglob("*.py"):
        t = f.read_text()
        assert "import oracle" not in t and "from oracle" not in t
