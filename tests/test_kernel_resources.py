"""Register and LDS budgets of every kernel, from the compiler's own resource
report (hipcc -Rpass-analysis=kernel-resource-usage on the library's device
code).  CPU only: the code is cross-compiled for gfx950 here.

A spill (scratch memory per lane) in a GEMM kernel turns register reads into
memory traffic inside the K loop; none of the kernels may have one.  The
default kernels must also keep the occupancy their tiling was designed for:
it is what hides the latency of the LDS reads and the global->LDS copies."""

from __future__ import annotations

import pytest

from dense_fp32_tiled_amd import build


@pytest.fixture(scope="module")
def report():
    return build.resource_report()


def kernels(report, fragment):
    return {k: v for k, v in report.items() if fragment in k}


def test_every_kernel_is_spill_free(report):
    assert len(report) >= 30
    spilled = {k: v["scratch"] for k, v in report.items() if v.get("scratch", 0) != 0}
    assert not spilled, spilled


def test_default_kernels_keep_their_occupancy(report):
    # fp32 256x256x32 pipelined kernel (AUTO for large problems): one 8-wave workgroup per CU, 128 KiB of LDS
    fp32_big = {k: v for k, v in kernels(report, "MfmaCfgILi256ELi256ELi32ELi128ELi64ELi2ELi32E").items()
                if "EEELi4ELi1ELi1ELb1ELi0ELi0EE" in k}
    assert len(fp32_big) == 1
    (r,) = fp32_big.values()
    assert r["occupancy"] == 2 and r["lds"] == 128 * 1024
    # its non-pipelined 256x256x16 ablation: same occupancy, 64 KiB of LDS
    fp32_plain = kernels(report, "MfmaCfgILi256ELi256ELi16ELi128ELi64ELi2ELi32ENS_10TileLayoutILi0ELi4ELi2ELi3EEENS2_"
                                 "ILi0ELi0ELi0ELi0EEELi4ELi1ELi1ELb0ELi0ELi0EE")
    assert len(fp32_plain) == 1
    (r,) = fp32_plain.values()
    assert r["occupancy"] == 2 and r["lds"] == 64 * 1024
    # fp32 256x128 direct-copy kernel (AUTO when 256x256 tiles round badly): 4 waves per SIMD = two workgroups
    fp32_default = kernels(report, "MfmaCfgILi256ELi128ELi16ELi64ELi64ELi2ELi32ENS_10TileLayoutILi0ELi4ELi2ELi3EEENS2_"
                                   "ILi0ELi0ELi0ELi0EEELi4ELi1ELi1ELb0ELi0ELi0EE")
    assert len(fp32_default) == 1
    (r,) = fp32_default.values()
    assert r["occupancy"] == 4 and r["lds"] == 48 * 1024
    # fp32 64x64x32 direct-copy kernel (AUTO for small grids): at least 4 waves per SIMD with 16-byte copies,
    # at least 2 with 4-byte copies; 32 KiB of LDS
    fp32_small = {k: v for k, v in kernels(report, "MfmaCfgILi64ELi64ELi32ELi32ELi32ELi2ELi32E").items()
                  if "16gemm_mfma_kernel" in k}
    vec4 = [v for k, v in fp32_small.items() if "EEELi4ELi1ELi1ELb0ELi0ELi8EE" in k]
    vec1 = [v for k, v in fp32_small.items() if "EEELi1ELi1ELi1ELb0ELi0ELi8EE" in k]
    assert len(vec4) == 1 and len(vec1) == 1
    assert vec4[0]["occupancy"] >= 4 and vec1[0]["occupancy"] >= 2
    assert vec4[0]["lds"] == vec1[0]["lds"] == 32 * 1024
    # K-split kernels: one workgroup (8 or 16 waves) per CU at least
    ksplit = kernels(report, "gemm_mfma_ksplit_kernel")
    assert len(ksplit) == 16  # 4 variants x 4 copy-width forms
    assert all(v["occupancy"] >= 2 and v["lds"] <= 160 * 1024 for v in ksplit.values())
    # bf16 / fp16 256x256x64 (AUTO for large problems): 2 waves per SIMD, 128 KiB of LDS
    mixed_default = kernels(report, "MixedCfgILi0ELi256ELi256ELi64E")
    assert mixed_default and all(v["occupancy"] == 2 and v["lds"] == 128 * 1024 for v in mixed_default.values())


def test_lds_fits_the_cu(report):
    for name, v in report.items():
        assert v.get("lds", 0) <= 160 * 1024, name
