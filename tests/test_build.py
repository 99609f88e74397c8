"""The build's resource check (CPU only): remarks parsed per kernel, and the
spill rule applied."""
from exact_io_aware_38_amd import build

REMARKS = """x.hip:93:1: remark: Function Name: _ZN4attn12_GLOBAL__N_118fwd_prefill_kernelILi128ENS_7NoTableELb0EEEvNS0_7FwdArgsET0_ [-Rpass-analysis=kernel-resource-usage]
x.hip:93:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:93:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:93:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:93:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
x.hip:414:1: remark: Function Name: _ZN4attn12_GLOBAL__N_116fwd_split_kernelILi128EEEvNS0_7FwdArgsE [-Rpass-analysis=kernel-resource-usage]
x.hip:414:1: remark:     VGPRs: 249 [-Rpass-analysis=kernel-resource-usage]
x.hip:414:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_remarks_are_parsed():
    r = build._resources(REMARKS)
    assert len(r) == 2
    assert "fwd_prefill_kernelILi128" in r[0]["kernel"] and "fwd_split_kernelILi128" in r[1]["kernel"]
    assert r[0]["VGPRs"] == 256 and r[0]["AGPRs"] == 0 and r[0]["ScratchSize"] == 0 and r[0]["Occupancy"] == 2
    assert r[1]["VGPRs"] == 249 and r[1]["ScratchSize"] == 12


def test_only_listed_kernels_may_spill():
    r = build._resources(REMARKS)
    spilling = [k["kernel"] for k in r if k.get("ScratchSize", 0) > 0
                and not any(a in k["kernel"] for a in build.SCRATCH_ALLOWED)]
    assert spilling == [r[1]["kernel"]]                 # the split kernel is not on the list
    assert not any(a in r[0]["kernel"] for a in build.SCRATCH_ALLOWED)   # the benchmarked prefill is not either


def test_calibration_library_is_separate_and_exports_its_entry():
    """The benchmark's calibration kernels (MFMA ceiling, matrix/vector
    co-issue) live in their own library, so libattn.so exports only the
    attention entry points."""
    import ctypes
    import os
    import subprocess
    assert os.path.exists(build.CALIB_LIB), "run __graft_entry__.build() first"
    lib = ctypes.CDLL(build.CALIB_LIB)
    for name in ("calib_mfma_bf16", "calib_coissue"):
        assert hasattr(lib, name)
    syms = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True, text=True).stdout
    assert "calib_" not in syms
