"""Host logic of the benchmark (CPU only): the work each kernel is credited
with, the roofline arithmetic, the counter staleness rule, the stats
summary, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_nominal_flops_match_the_formula():
    # 4 B H Sq Sk d, halved for causal
    assert bench.nominal_fwd_flops(2, 32, 8192, 8192, 128, 1) == 2 * 32 * 8192 * 8192 * 128 * 2
    assert bench.nominal_fwd_flops(1, 1, 256, 256, 64, 0) == 4 * 256 * 256 * 64


def test_kernel_work_per_launch():
    w = synth.get_workload("train_causal_d128")
    fwd = bench.nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    assert bench.kernel_work("fwd_prefill_bf16", w) == {"bound": "mfma", "flops": fwd}
    assert bench.kernel_work("bwd_dkdv", w)["flops"] == 2 * fwd          # S, dP, dV, dK: 8 d per pair
    assert bench.kernel_work("bwd_dq", w)["flops"] == 0.5 * fwd          # dQ only: 2 d per pair
    assert bench.kernel_work("fwd_fp8", w)["peak"] == bench.PEAK_FP8_TFLOPS
    d = synth.get_workload("gqa_decode")
    kv = 2 * d.B * d.Hkv * d.Sk * d.d
    assert bench.kernel_work("fwd_split_bf16", d)["bytes"] == 2 * kv + d.B * d.Hq * d.Sq * d.d * 2
    f8 = bench.kernel_work("fwd_fp8_split", d)["bytes"]
    assert f8 == pytest.approx(kv * (1 + 1 / 32) + d.B * d.Hq * d.Sq * d.d * (1 + 1 / 32))


def test_roofline_arithmetic():
    w = synth.get_workload("long_causal_d128")
    r = bench.roofline("fwd_prefill_bf16", w, 1.0)
    flops = bench.nominal_fwd_flops(w.B, w.Hq, w.Sq, w.Sk, w.d, w.causal)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.PEAK_BF16_TFLOPS
    assert r["achieved"] == pytest.approx(flops / 1e-3 / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    d = synth.get_workload("gqa_decode")
    r = bench.roofline("fwd_split_bf16", d, 0.5)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["achieved"] == pytest.approx(bench.kernel_work("fwd_split_bf16", d)["bytes"] / 0.5e-3 / 1e9, rel=1e-4)


def test_traffic_is_null_for_stale_or_missing_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_for("fwd_fp8", "long_causal_d128_mxfp8") is None        # missing
    path = tmp_path / "counters_fwd_fp8__long_causal_d128_mxfp8.json"
    path.write_text(json.dumps({"source_sha": bench.source_hash("fwd_fp8"), "hbm_bytes_per_launch": 123}))
    assert bench.traffic_for("fwd_fp8", "long_causal_d128_mxfp8") == 123           # current
    path.write_text(json.dumps({"source_sha": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_for("fwd_fp8", "long_causal_d128_mxfp8") is None        # kernel changed since


def test_stats_summary_table(tmp_path):
    csv_path = tmp_path / "kernel_stats.csv"
    csv_path.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                        '"void attn::(anonymous namespace)::fwd_fp8_kernel<128>(attn::(anonymous namespace)::Fp8Args)",'
                        '25,23157637,926305.48,96.47,844962,1038135,56008.9\n'
                        '"_ZN4attn12_GLOBAL__N_120mx_quant_rows_kernelEPKDF16bPhS3_x",14,489691,34977.9,2.04,33396,37114,1047.8\n')
    out = tmp_path / "s.md"
    bench.summarize_stats(str(csv_path), "t", str(out), "cmd")
    text = out.read_text()
    assert "| fwd_fp8_kernel<128> | 25 | 926.3 | 845.0 | 1038.1 | 96.5% |" in text
    assert "| mx_quant_rows_kernel | 14 | 35.0 |" in text
    assert "cmd" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_spread_statistics():
    s = bench.spread([1.0, 2.0, 3.0, 4.0, 100.0])
    assert s["median_ms"] == 3.0 and s["min_ms"] == 1.0 and s["max_ms"] == 100.0 and s["n"] == 5
    assert s["p10_ms"] == pytest.approx(1.4) and s["p90_ms"] == pytest.approx(61.6)


def test_shader_counter_summary(tmp_path):
    # two passes over the same kernel, as two rocprofv3 --pmc runs write them
    hdr = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
           '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count",'
           '"SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')
    k = '"void attn::(anonymous namespace)::bwd_dkdv_kernel<128, true>(attn::(anonymous namespace)::BwdArgs)"'
    a = tmp_path / "a"
    b = tmp_path / "b"
    a.mkdir()
    b.mkdir()
    # 1 ms dispatch; 8 XCDs x 2e6 cycles -> 2 GHz; MFMA busy half of 1024 SIMDs x 2e6 cycles
    (a / "c_counter_collection.csv").write_text(
        hdr + f'1,1,"A",1,1,1,1,1,{k},512,0,0,8,0,16,"GRBM_GUI_ACTIVE",16000000,0,1000000\n'
        f'1,1,"A",1,1,1,1,1,{k},512,0,0,8,0,16,"SQ_VALU_MFMA_BUSY_CYCLES",1024000000,0,1000000\n')
    (b / "c_counter_collection.csv").write_text(
        hdr + f'1,1,"A",1,1,1,1,1,{k},512,0,0,8,0,16,"SQ_INSTS_VALU_TRANS_F32",25,0,1000000\n'
        f'1,1,"A",1,1,1,1,1,{k},512,0,0,8,0,16,"SQ_INSTS_VALU",100,0,1000000\n'
        f'1,1,"A",1,1,1,1,1,{k},512,0,0,8,0,16,"SQ_INSTS_VALU_MFMA_MOPS_BF16",2000000000,0,1000000\n')
    out = bench.summarize_pmc("w", "title", [str(a), str(b)], "cmd", out_md=str(tmp_path / "p.md"))
    text = open(out).read()
    assert "## bwd_dkdv_kernel<128, true>" in text
    assert "| clock (GHz) | 2.000 |" in text
    assert "| MFMA busy (%) | 50.0 |" in text
    assert "| TRANS share of VALU instructions (%) | 25.0 |" in text
    assert "| executed MFMA work, bf16 (TFLOP) | 1.0240 |" in text


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """Counters stay valid across comment edits and go stale on code edits."""
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    for f in bench.KERNEL_SOURCES["fwd_f32"]:
        (tmp_path / f).write_text("int x = 1; // note\n")
    h0 = bench.source_hash("fwd_f32")
    (tmp_path / "fwd_f32.hip").write_text("/* a block\n   comment */ int  x = 1;   // another note\n")
    assert bench.source_hash("fwd_f32") == h0
    (tmp_path / "fwd_f32.hip").write_text("int x = 2; // note\n")
    assert bench.source_hash("fwd_f32") != h0
