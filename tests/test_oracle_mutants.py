"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pins catch every one of them.

Each mutant is the oracle's own source with one textual change, executed as a
fresh module; the pins of test_oracle are then run against it and at least one
must fail.
"""
import inspect
import types

import pytest

import oracle.attention as attn_mod
import test_oracle as pins

MUTANTS = {
    "online_drops_rescale_of_u": ("u = a[:, None] * u + p @ v[b, hk, start:stop]",
                                  "u = u + p @ v[b, hk, start:stop]"),
    "online_drops_rescale_of_l": ("l = a * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    "online_forgets_final_division": ("o[b, h, ok] = u[ok] / l[ok, None]", "o[b, h, ok] = u[ok]"),
    "forward_mask_not_applied": ("            s = np.where(vis, s, -np.inf)\n            m = s.max(axis=1, initial=-np.inf)          # row max",
                                 "            m = s.max(axis=1, initial=-np.inf)          # row max"),
    "forward_lse_without_log": ("            lse[b, h, ok] = m[ok] + np.log(l[ok])\n    return o, lse\n\n\ndef attention_backward",
                                "            lse[b, h, ok] = m[ok] + l[ok]\n    return o, lse\n\n\ndef attention_backward"),
    "bottom_right_offset_sign": ("(i[:, None] + (Sk - Sq))", "(i[:, None] + (Sq - Sk))"),
    "top_left_strict_inequality": ("return j[None, :] <= i[:, None]", "return j[None, :] < i[:, None]"),
    "gqa_interleaved_heads": ("            hk = h // g\n            s = c * (q[b, h] @ k[b, hk].T)              # [n, Sk]",
                              "            hk = h % Hkv\n            s = c * (q[b, h] @ k[b, hk].T)              # [n, Sk]"),
    "backward_jacobian_sign": ("ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])"),
    "backward_dq_missing_scale": ("dq[b, h] = c * (ds @ k[b, hk])", "dq[b, h] = ds @ k[b, hk]"),
    "backward_dk_transposed_operand": ("dk[b, hk] += c * (ds.T @ q[b, h])", "dk[b, hk] += c * (p.T @ q[b, h])"),
    "backward_dv_drops_probabilities": ("dv[b, hk] += pz.T @ do[b, h]", "dv[b, hk] += vis.T @ do[b, h]"),
    "dropout_dv_without_mask": ("pz = p if Z is None else p * Z[b, h]", "pz = p"),
    "dropout_dp_without_mask": ("                dp = dp * Z[b, h]", "                dp = dp"),
    "dropout_rows_and_keys_swapped": ("full = byte.transpose(0, 1, 3, 2, 4)", "full = byte.transpose(0, 1, 2, 3, 4)"),
    "dropout_kept_values_not_rescaled": ("keep.astype(np.float64) / (1.0 - thr / 256.0)", "keep.astype(np.float64)"),
    "varlen_keys_cut_at_query_offsets": ("        ks = slice(cu_k[b], cu_k[b + 1])\n        ob, lb",
                                         "        ks = slice(cu_q[b], cu_q[b + 1])\n        ob, lb"),
    "varlen_mask_on_packed_rows": ("causal=causal, scale=scale)\n        o[:, qs] = ob[0]",
                                   "causal=causal, scale=scale, rows=list(range(qs.start, qs.stop)),\n"
                                   "                                   Sq=cu_q[-1])\n        o[:, qs] = ob[0]"),
    "varlen_backward_dk_overwritten_by_dv": ('        dk[:, ks] = g["dk"][0]', '        dk[:, ks] = g["dv"][0]'),
    "varlen_backward_keys_cut_at_query_offsets": ("        ks = slice(cu_k[b], cu_k[b + 1])\n        g = attention_backward",
                                                  "        ks = slice(cu_q[b], cu_q[b + 1])\n        g = attention_backward"),
    "merge_wrong_weight": ("wb[live] = np.exp(lse_b[live] - M[live])", "wb[live] = np.exp(lse_a[live] - M[live])"),
}

# (pin function, kwargs) pairs run against each mutant
PIN_CALLS = [
    (pins.test_worked_example_states_and_output, {}),
    (pins.test_tile_invariance, {"causal": 1, "tile": 3}),
    (pins.test_tile_invariance, {"causal": 2, "tile": 8}),
    (pins.test_single_visible_key, {"causal": 1}),
    (pins.test_zero_keys_give_mean_of_visible_values, {"causal": 2}),
    (pins.test_forward_matches_torch_sdpa_fp64, {"causal": 1, "gqa": True}),
    (pins.test_forward_matches_torch_sdpa_fp64, {"causal": 2, "gqa": False}),
    (pins.test_fully_masked_rows_strict_and_defined, {}),
    (pins.test_merge_states_equals_single_pass, {}),
    (pins.test_central_differences_masked_2x3x2, {}),
    (pins.test_backward_matches_torch_autograd_fp64, {"causal": 1, "shape": (2, 4, 2, 5, 9, 8)}),
    (pins.test_varlen_matches_block_diagonal_softmax, {"causal": 1}),
    (pins.test_varlen_matches_block_diagonal_softmax, {"causal": 2}),
    (pins.test_varlen_central_differences, {"causal": 2}),
    (pins.test_varlen_backward_matches_autograd_block_diagonal, {}),
    (pins.test_dropout_mask_layout_rate_and_streams, {}),
    (pins.test_dropout_central_differences, {}),
    (pins.test_dropout_matches_torch_autograd_fp64, {"causal": 2}),
]

_NAMES = ["attention_forward", "attention_backward", "online_softmax_forward",
          "merge_states", "visible_mask", "FullyMaskedRowError", "attention_forward_varlen",
          "attention_backward_varlen", "philox4x32_10", "dropout_threshold", "dropout_keep_mask"]


def _mutant_module(old, new):
    src = inspect.getsource(attn_mod)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    mod = _mutant_module(*MUTANTS[name])
    for n in _NAMES:
        monkeypatch.setattr(pins, n, getattr(mod, n))
    failures = 0
    for fn, kw in PIN_CALLS:
        try:
            fn(**kw)
        except (Exception, pytest.fail.Exception):   # an assertion, pytest.raises, or a crash
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_all_pins(monkeypatch):
    mod = _mutant_module("import math", "import math")
    for n in _NAMES:
        monkeypatch.setattr(pins, n, getattr(mod, n))
    for fn, kw in PIN_CALLS:
        fn(**kw)


# ------------------------------------------------------------------ FP8 oracle
import oracle.fp8 as fp8_mod          # noqa: E402
import test_oracle_fp8 as fp8_pins    # noqa: E402

FP8_MUTANTS = {
    "e4m3_exponent_bias_8": ("np.exp2(ex.astype(np.float64) - 7.0)", "np.exp2(ex.astype(np.float64) - 8.0)"),
    "e4m3_subnormals_one_binade_low": ("man / 8.0 * 2.0 ** -6", "man / 8.0 * 2.0 ** -7"),
    "encode_ties_away_from_zero": ("q = np.rint(a / step)", "q = np.floor(a / step + 0.5)"),
    "encode_subnormal_floor_off_by_one": ("E = np.maximum(E, -6.0)", "E = np.maximum(E, -7.0)"),
    "block_exponent_saturating_floor_rule": ("e = E - 9 + (1 if f > 0.875 else 0)", "e = E - 9"),
    "block_exponent_wasteful_by_one": ("e = E - 9 + (1 if f > 0.875 else 0)", "e = E - 8 + (1 if f > 0.875 else 0)"),
    "dequantize_scale_bias_128": ("np.exp2(sm.astype(np.float64) - 127.0)", "np.exp2(sm.astype(np.float64) - 128.0)"),
    "fp8_attention_uses_padding_keys": ("v = np.swapaxes(mx_dequantize(vt8, vs, axis=-1), -1, -2)[:, :, :Sk, :]",
                                        "v = np.swapaxes(mx_dequantize(vt8, vs, axis=-1), -1, -2)[:, :, -Sk:, :]"),
}

FP8_PINS = [getattr(fp8_pins, n) for n in dir(fp8_pins) if n.startswith("test_")]


def _fp8_mutant_module(old, new):
    src = inspect.getsource(fp8_mod)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "<oracle_fp8_mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_pins_catch_mutant(name, monkeypatch):
    monkeypatch.setattr(fp8_pins, "fp8", _fp8_mutant_module(*FP8_MUTANTS[name]))
    failures = 0
    for fn in FP8_PINS:
        try:
            fn()
        except (Exception, pytest.fail.Exception):
            failures += 1
    assert failures > 0, f"no FP8 pin caught mutant {name}"


def test_fp8_unmutated_copy_passes_all_pins(monkeypatch):
    monkeypatch.setattr(fp8_pins, "fp8", _fp8_mutant_module("import math", "import math"))
    for fn in FP8_PINS:
        fn()
