"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments before touching any device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_38_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = 0x1000          # non-NULL pointer value that is never dereferenced: validation fails first


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = attn.lib()
    names = _declared()
    assert {"attn_fwd", "attn_bwd", "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes",
            "attn_strerror", "attn_last_dispatch"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libattn.so does not export {n}"


def test_strerror_covers_every_status():
    codes = {0: "success", -1: "NULL", -2: "shape", -3: "multiple", -4: "head dim", -5: "dtype",
             -6: "causal", -7: "workspace", -8: "HIP", -9: "scale", -10: "dropout", -11: "misaligned", -12: "scratch"}
    for c, word in codes.items():
        assert word.lower() in attn.strerror(c).lower()
    assert "unknown" in attn.strerror(-99)


def _fwd(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64,
             causal=0, scale=0.125, dtype=attn.ATTN_BF16, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return attn.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                               a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"], a["ws"],
                               a["ws_bytes"], a["stream"])


def _bwd(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=4,
             Hkv=2, Sq=16, Sk=16, d=64, causal=0, scale=0.125, dtype=attn.ATTN_BF16, ws=None,
             ws_bytes=0, stream=None)
    a.update(over)
    return attn.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                               a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["causal"],
                               a["scale"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, -1), ({"k": None}, -1), ({"v": None}, -1), ({"o": None}, -1),
    ({"B": 0}, -2), ({"Hq": 0}, -2), ({"Hkv": 0}, -2), ({"Sq": 0}, -2), ({"Sk": -1}, -2),
    ({"B": 1 << 20, "Hq": 1 << 10, "Hkv": 1 << 10}, -2),
    ({"Hq": 2, "Sk": 1 << 24}, -2), ({"Hq": 2, "Sq": 1 << 24}, -2),   # per-head byte ranges are 32-bit
    ({"Hq": 6, "Hkv": 4}, -3), ({"d": 96}, -4), ({"d": 256}, -4), ({"dtype": 7}, -5),
    ({"causal": 3}, -6), ({"causal": -1}, -6), ({"scale": 0.0}, -9), ({"scale": -1.0}, -9),
    ({"scale": float("nan")}, -9), ({"scale": float("inf")}, -9),
    # the decode-shaped calls (here Hq/Hkv * Sq <= 32) need a workspace for the per-split partials
    ({"Sq": 1, "Sk": 4096}, -7),
    ({"ws": FAKE, "ws_bytes": 16}, -7),
])
def test_fwd_validation(over, code):
    assert _fwd(**over) == code


@pytest.mark.parametrize("over,code", [
    ({"lse": None}, -1), ({"do": None}, -1), ({"dq": None}, -1), ({"dk": None}, -1), ({"dv": None}, -1),
    ({"o": None}, -1), ({"Sq": 0}, -2), ({"Hq": 3, "Hkv": 2}, -3), ({"d": 32}, -4),
    ({"dtype": attn.ATTN_F32}, -5), ({"causal": 5}, -6), ({"scale": 0.0}, -9),
    ({}, -7),                                   # no workspace
    ({"ws": FAKE, "ws_bytes": 8}, -7),          # too small
])
def test_bwd_validation(over, code):
    assert _bwd(**over) == code


def test_workspace_queries():
    # bf16 prefill reads K and V in place; decode (4 query rows per KV head) keeps the split partials
    assert attn.fwd_workspace_bytes(2, 32, 32, 8192, 8192, 128, 1, attn.ATTN_BF16) == 0
    assert attn.fwd_workspace_bytes(1, 4, 2, 100, 70, 64, 0, attn.ATTN_BF16) == 0
    n = attn.fwd_workspace_bytes(16, 32, 8, 1, 32768, 128, 0, attn.ATTN_BF16)
    assert n >= 16 * 32 * 129 * 4
    assert attn.fwd_workspace_bytes(1, 1, 1, 1, 100, 64, 0, attn.ATTN_F32) == 0
    assert attn.fwd_workspace_bytes(0, 1, 1, 1, 1, 64, 0, attn.ATTN_BF16) == 0     # invalid -> 0
    rows = 1 * 32 * 8192
    assert attn.bwd_workspace_bytes(1, 32, 32, 8192, 8192, 128, 1, attn.ATTN_BF16) >= 2 * 4 * rows
    assert attn.bwd_workspace_bytes(1, 32, 32, 8192, 8192, 128, 1, attn.ATTN_F32) == 0


def test_dispatch_record_is_empty_before_any_call():
    import threading
    out = {}
    th = threading.Thread(target=lambda: out.setdefault("d", attn.last_dispatch()))
    th.start()
    th.join()
    assert out["d"] == ""
    assert attn.lib().attn_last_dispatch(None, 8) == -1


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(attn, "_lib", None)
    monkeypatch.setattr(attn, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        attn.lib()


# ---------------------------------------------------------------- packed variable-length batches
def _ints(vals):
    return None if vals is None else (ctypes.c_int * len(vals))(*vals)


def _fwd_varlen(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cq=[0, 5, 12], ck=[0, 7, 7], B=2, Hq=4, Hkv=2,
             d=64, causal=1, scale=0.125, dtype=attn.ATTN_BF16, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return attn.lib().attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], _ints(a["cq"]),
                                      _ints(a["ck"]), a["B"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                      a["scale"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def _bwd_varlen(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             cq=[0, 5, 12], ck=[0, 7, 7], B=2, Hq=4, Hkv=2, d=64, causal=1, scale=0.125,
             dtype=attn.ATTN_BF16, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return attn.lib().attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                      a["dv"], _ints(a["cq"]), _ints(a["ck"]), a["B"], a["Hq"], a["Hkv"],
                                      a["d"], a["causal"], a["scale"], a["dtype"], a["ws"], a["ws_bytes"],
                                      a["stream"])


@pytest.mark.parametrize("over,code", [
    ({"cq": None}, -1), ({"ck": None}, -1),
    ({"q": None}, -1), ({"o": None}, -1), ({"k": None}, -1),
    ({"B": 0, "cq": [0], "ck": [0]}, -2),
    ({"cq": [1, 5, 12]}, -2), ({"ck": [0, 7, 3]}, -2),          # must start at 0 and never decrease
    ({"cq": [0, 1 << 30, (1 << 30) + 2]}, -2),                 # Hq * total_q past 2^31
    ({"Hq": 2, "ck": [0, 1 << 24, 1 << 24]}, -2),              # one sequence at the per-head limit
    ({"Hq": 6, "Hkv": 4}, -3), ({"d": 96}, -4), ({"dtype": 3}, -5), ({"causal": 3}, -6),
    ({"scale": 0.0}, -9),
    ({"cq": [0, 1, 2], "ck": [0, 4096, 8192]}, -7),            # decode-shaped sequences need a workspace
])
def test_fwd_varlen_validation(over, code):
    assert _fwd_varlen(**over) == code


@pytest.mark.parametrize("over,code", [
    ({"cq": None}, -1), ({"lse": None}, -1), ({"dq": None}, -1), ({"dk": None}, -1),
    ({"cq": [0, 5, 4]}, -2), ({"Hq": 3, "Hkv": 2}, -3), ({"d": 32}, -4),
    ({"dtype": attn.ATTN_F32}, -5), ({"causal": -1}, -6), ({"scale": float("nan")}, -9),
    ({}, -7), ({"ws": FAKE, "ws_bytes": 8}, -7),
])
def test_bwd_varlen_validation(over, code):
    assert _bwd_varlen(**over) == code


def test_varlen_with_only_empty_sequences_launches_nothing():
    # every sequence empty: nothing to read or write, so NULL tensors are fine
    none = dict(q=None, k=None, v=None, o=None, lse=None, cq=[0, 0, 0], ck=[0, 0, 0])
    assert _fwd_varlen(**none) == 0
    assert attn.last_dispatch().startswith("attn_fwd_varlen: 0 sequences of 2 launched")
    assert _bwd_varlen(do=None, dq=None, dk=None, dv=None, **none) == 0
    assert attn.last_dispatch().startswith("attn_bwd_varlen: 0 sequences of 2 launched")
    # queries without keys still need q and o
    assert _fwd_varlen(q=None, cq=[0, 3, 3], ck=[0, 0, 0]) == -1


def test_varlen_workspace_queries():
    bf = attn.ATTN_BF16
    cq, ck = [0, 1, 2, 3], [0, 32768, 40000, 72768]
    n = attn.fwd_varlen_workspace_bytes(cq, ck, 32, 8, 128, 0, bf)
    assert n == max(attn.fwd_workspace_bytes(1, 32, 8, 1, s, 128, 0, bf) for s in (32768, 7232, 32768))
    assert n > 0
    assert attn.fwd_varlen_workspace_bytes([0, 100, 300], [0, 100, 300], 4, 4, 64, 1, bf) == 0
    lens = [100, 0, 2000]
    cu = [0, 100, 100, 2100]
    nb = attn.bwd_varlen_workspace_bytes(cu, cu, 8, 2, 128, 1, bf)
    # lse2 and D (two floats) for every query row of every head, each sequence padded to 64 rows
    rows = sum((s + 63) // 64 * 64 for s in lens)
    assert nb == (rows * 8 * 2 * 4 + 255) // 256 * 256
    assert attn.bwd_varlen_workspace_bytes(cu, cu, 8, 2, 128, 1, attn.ATTN_F32) == 0
    assert attn.fwd_varlen_workspace_bytes([0, 5, 3], [0, 5, 6], 1, 1, 64, 0, bf) == 0   # invalid -> 0
    with pytest.raises(ValueError):
        attn.fwd_varlen_workspace_bytes([0, 5], [0, 5, 6], 1, 1, 64, 0, bf)


# ---------------------------------------------------------------- dropout
def _fwd_drop(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64, causal=1,
             scale=0.125, p=0.1, seed=1, offset=0, stream=None)
    a.update(over)
    return attn.lib().attn_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                       a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["p"], a["seed"],
                                       a["offset"], a["stream"])


def _bwd_drop(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=4, Hkv=2,
             Sq=16, Sk=16, d=64, causal=1, scale=0.125, p=0.1, seed=1, offset=0, ws=None, ws_bytes=0,
             stream=None)
    a.update(over)
    return attn.lib().attn_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                       a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["causal"],
                                       a["scale"], a["p"], a["seed"], a["offset"], a["ws"], a["ws_bytes"],
                                       a["stream"])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, -1), ({"v": None}, -1), ({"Sq": 0}, -2), ({"Hq": 3}, -3), ({"d": 80}, -4),
    ({"causal": 4}, -6), ({"scale": 0.0}, -9),
    ({"p": -0.01}, -10), ({"p": 1.0}, -10), ({"p": 0.999}, -10), ({"p": float("nan")}, -10),
])
def test_fwd_dropout_validation(over, code):
    assert _fwd_drop(**over) == code


@pytest.mark.parametrize("over,code", [
    ({"lse": None}, -1), ({"dk": None}, -1), ({"Sk": -2}, -2), ({"p": 2.0}, -10), ({"p": float("inf")}, -10),
    ({}, -7), ({"ws": FAKE, "ws_bytes": 4}, -7),
])
def test_bwd_dropout_validation(over, code):
    assert _bwd_drop(**over) == code


def test_dropout_mask_validation():
    L = attn.lib()
    assert L.attn_dropout_mask(None, 1, 1, 4, 4, 0.1, 1, 0, None) == -1
    assert L.attn_dropout_mask(FAKE, 0, 1, 4, 4, 0.1, 1, 0, None) == -2
    assert L.attn_dropout_mask(FAKE, 1, 1, 4, 4, 1.5, 1, 0, None) == -10
    assert "dropout" in attn.strerror(-10)


# ---------------------------------------------------------------- FP8
def _fwd_fp8(**over):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, vt=FAKE, vs=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=16,
             Sk=16, d=128, causal=1, scale=0.125, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    return attn.lib().attn_fwd_fp8(a["q"], a["qs"], a["k"], a["ks"], a["vt"], a["vs"], a["o"], a["lse"], a["B"],
                                   a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["ws"],
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, -1), ({"qs": None}, -1), ({"k": None}, -1), ({"ks": None}, -1), ({"vt": None}, -1),
    ({"vs": None}, -1), ({"o": None}, -1), ({"Sq": 0}, -2), ({"Sk": -1}, -2), ({"Hq": 2, "Sk": 1 << 24}, -2),
    ({"Hq": 3}, -3), ({"d": 64}, -4), ({"d": 96}, -4), ({"causal": 3}, -6), ({"scale": 0.0}, -9),
    # decode-shaped calls (Hq/Hkv * Sq <= 32) split the keys and need the partials workspace
    ({"Sq": 1, "Sk": 4096}, -7), ({"Sq": 1, "Sk": 4096, "ws": FAKE, "ws_bytes": 8}, -7),
])
def test_fwd_fp8_validation(over, code):
    assert _fwd_fp8(**over) == code


def test_fwd_fp8_workspace_query():
    # prefill-shaped: none; decode-shaped: the bf16 split path's partials, same rule
    assert attn.fwd_fp8_workspace_bytes(1, 4, 2, 256, 256, 128, 1) == 0
    n = attn.fwd_fp8_workspace_bytes(16, 32, 8, 1, 32768, 128, 0)
    assert n > 0 and n == attn.fwd_workspace_bytes(16, 32, 8, 1, 32768, 128, 0, attn.ATTN_BF16)
    assert attn.fwd_fp8_workspace_bytes(16, 32, 8, 1, 32768, 64, 0) == 0        # d = 64 is not built


def test_mxfp8_quantizer_validation():
    L = attn.lib()
    assert L.attn_mxfp8_quantize_rows(None, FAKE, FAKE, 4, 128, None) == -1
    assert L.attn_mxfp8_quantize_rows(FAKE, FAKE, FAKE, -1, 128, None) == -2
    assert L.attn_mxfp8_quantize_rows(FAKE, FAKE, FAKE, 4, 64, None) == -4
    assert L.attn_mxfp8_quantize_rows(None, None, None, 0, 128, None) == 0      # nothing to do
    assert L.attn_mxfp8_quantize_vt(FAKE, None, FAKE, 2, 100, 128, None) == -1
    assert L.attn_mxfp8_quantize_vt(FAKE, FAKE, FAKE, 0, 100, 128, None) == -2
    assert L.attn_mxfp8_quantize_vt(FAKE, FAKE, FAKE, 2, 1 << 24, 128, None) == -2
    assert L.attn_mxfp8_quantize_vt(FAKE, FAKE, FAKE, 2, 100, 96, None) == -4
    assert [attn.fp8_padded_keys(n) for n in (0, 1, 64, 65, 2000)] == [0, 64, 64, 128, 2048]
    assert L.attn_fp8_padded_keys(-1) == -2


# ---------------------------------------------------------------- pointer alignment
ODD16 = FAKE + 8        # 8-byte but not 16-byte aligned
ODD4 = FAKE + 2         # not even 4-byte aligned


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "ws"])
def test_fwd_rejects_misaligned_tensors(name):
    over = {name: ODD16}
    if name == "ws":
        over["ws_bytes"] = 1 << 20
    assert _fwd(**over) == -11
    assert _fwd(lse=ODD4) == -11
    assert _fwd(lse=FAKE + 4) != -11      # lse needs only 4 bytes


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "do", "dq", "dk", "dv", "ws"])
def test_bwd_rejects_misaligned_tensors(name):
    assert _bwd(**{name: ODD16, "ws_bytes": 1 << 20} if name == "ws" else {name: ODD16}) == -11
    assert _bwd(lse=ODD4) == -11


def test_other_entry_points_reject_misaligned_tensors():
    assert _fwd_varlen(q=ODD16) == -11
    assert _bwd_varlen(dk=ODD16) == -11
    assert _fwd_drop(v=ODD16) == -11
    assert _bwd_drop(dq=ODD16) == -11
    assert _fwd_fp8(k=ODD16) == -11
    assert _fwd_fp8(ks=ODD4) == -11
    assert _fwd_fp8(ks=FAKE + 4) != -11    # scale arrays need only 4 bytes
    L = attn.lib()
    assert L.attn_mxfp8_quantize_rows(ODD16, FAKE, FAKE, 4, 128, None) == -11
    assert L.attn_mxfp8_quantize_vt(FAKE, ODD16, FAKE, 2, 100, 128, None) == -11


class _FakeTensor:
    """Stands in for a GPU tensor in the binding's argument checks (no device needed)."""

    def __init__(self, ptr):
        self._ptr = ptr
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._ptr


def test_binding_checks_alignment_before_calling():
    attn._check(_FakeTensor(FAKE), "q")
    attn._check(_FakeTensor(FAKE + 4), "lse")
    with pytest.raises(ValueError, match="16-byte"):
        attn._check(_FakeTensor(ODD16), "q")
    with pytest.raises(ValueError, match="4-byte"):
        attn._check(_FakeTensor(ODD4), "lse")


# ---------------------------------------------------------------- forward on the static scratch
def _fwd_noalloc(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64,
             causal=0, scale=0.125, dtype=attn.ATTN_BF16, stream=None)
    a.update(over)
    return attn.lib().attn_fwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                       a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("over,code", [
    ({"q": None}, -1), ({"k": None}, -1), ({"B": 0}, -2), ({"Hq": 6, "Hkv": 4}, -3), ({"d": 96}, -4),
    ({"dtype": 7}, -5), ({"causal": 3}, -6), ({"scale": 0.0}, -9), ({"o": FAKE + 8}, -11),
    # decode whose split partials exceed the 16 MiB static scratch (checked before any HIP call)
    ({"B": 1024, "Hq": 32, "Hkv": 8, "Sq": 1, "Sk": 4096, "d": 128}, -12),
])
def test_fwd_noalloc_validation(over, code):
    assert _fwd_noalloc(**over) == code


def test_noalloc_scratch_limit_matches_the_workspace_query():
    # the limit is the same 16 MiB the header states; the training-size decode fits
    assert attn.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert 0 < attn.fwd_workspace_bytes(16, 32, 8, 1, 32768, 128, 0, attn.ATTN_BF16) <= attn.NOALLOC_SCRATCH_BYTES
    big = attn.fwd_workspace_bytes(1024, 32, 8, 1, 4096, 128, 0, attn.ATTN_BF16)
    assert big > attn.NOALLOC_SCRATCH_BYTES
