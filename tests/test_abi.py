"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before touching a device (CPU only)."""

from __future__ import annotations

import ctypes
import re
import subprocess
from pathlib import Path

import pytest

import dense_fp32_tiled_amd as dft

HEADER = Path(__file__).resolve().parent.parent / "include" / "dense_fp32_tiled.h"
PROBE_HEADER = HEADER.with_name("lds_probe.h")


def declared_functions(header: Path = HEADER) -> set[str]:
    text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def exported(lib: Path) -> set[str]:
    out = subprocess.run(["nm", "-D", "--defined-only", str(lib)], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_probe_library_exports_its_header(gemm_lib):
    from dense_fp32_tiled_amd import lds_probe

    assert declared_functions(PROBE_HEADER) == {"lds_probe_run", "probe_copy_f32", "probe_xcc_ids",
                                                "probe_dma_throughput", "probe_valu_fma",
                                                "probe_mfma_f32"}
    assert declared_functions(PROBE_HEADER) <= exported(lds_probe.PROBE_LIB)


def test_header_declares_the_binding_exports():
    assert declared_functions() == set(dft.EXPORTS)


def test_library_exports_every_declared_symbol(gemm_lib):
    missing = declared_functions() - exported(dft.LIB_PATH)
    assert not missing, f"declared but not exported: {missing}"
    for name in dft.EXPORTS:
        assert hasattr(gemm_lib, name)


def test_poison_build_exports_every_declared_symbol(gemm_lib):
    """The LDS-poison debug build is the same library: same entry points."""
    from dense_fp32_tiled_amd import build

    missing = declared_functions() - exported(build.POISON_LIB)
    assert not missing, f"declared but not exported by the poison build: {missing}"


def test_status_strings(gemm_lib):
    for st in range(-10, 1):
        s = dft.gemm_f32_status_string(st)
        assert s and s != "unknown status"
    assert dft.gemm_f32_status_string(12345) == "unknown status"


@pytest.mark.parametrize("variant", range(dft.VARIANT_COUNT))
def test_tile_config_is_consistent(variant, gemm_lib):
    c = dft.gemm_f32_tile_config(variant)
    assert c["variant"] == variant
    assert c["wave_size"] == 64
    assert c["a_row_stride"] == c["a_cols"] + c["a_pad"]
    assert c["b_row_stride"] == c["b_cols"] + c["b_pad"]
    assert c["a_stage_elems"] == c["a_rows"] * c["a_row_stride"]
    assert c["b_stage_elems"] == c["b_rows"] * c["b_row_stride"]
    # the pages' budget formula, on the physical (padded, staged) sizes
    assert c["lds_bytes"] == c["stages"] * (c["a_stage_elems"] + c["b_stage_elems"]) * 4
    assert c["lds_bytes"] <= 160 * 1024
    assert c["k_groups"] >= 1
    assert c["barriers_per_tile"] == (2 if c["stages"] == 1 else 1)
    if c["a_transposed"]:
        assert (c["a_rows"], c["a_cols"]) == (c["bk"], c["bm"])
        assert c["mfma_block"] == 0
    else:
        assert (c["a_rows"], c["a_cols"]) == (c["bm"], c["bk"])
        assert c["mfma_block"] in (16, 32)
        assert c["threads"] == (c["bm"] // c["tm"]) * (c["bn"] // c["tn"]) * 64 * c["k_groups"]
    assert (c["b_rows"], c["b_cols"]) == (c["bk"], c["bn"])
    assert c["vec_width"] in (1, 4)
    assert (c["a_row_stride"] % 4 == 0) and (c["b_row_stride"] % 4 == 0)
    if c["direct_to_lds"]:  # 16-byte copies into unpadded rows, two or more stages per group, matrix cores
        assert c["vec_width"] == 4 and c["a_pad"] == 0 and c["b_pad"] == 0
        assert c["stages"] == 2 * c["k_groups"]
        assert c["mfma_block"] in (16, 32)
    for t in "ab":
        unit, mask = c[f"{t}_swz_unit"], c[f"{t}_swz_mask"]
        if unit:  # a swizzle permutes whole 16-byte groups inside aligned blocks of a row
            assert unit % 4 == 0 and (mask & (mask + 1)) == 0
            assert c[f"{t}_cols"] % (unit * (mask + 1)) == 0


def test_tile_config_rejects(gemm_lib):
    with pytest.raises(dft.GemmError):
        dft.gemm_f32_tile_config(dft.VARIANT_COUNT)
    with pytest.raises(dft.GemmError):
        dft.gemm_f32_tile_config(-1)
    assert gemm_lib.gemm_f32_tile_config(0, None) == dft.GEMM_ERR_NULL


LAYOUT_KEYS = ("a_pad", "a_swz_unit", "a_swz_shift", "a_swz_mask", "b_pad", "b_swz_unit", "b_swz_shift",
               "b_swz_mask", "a_row_stride", "b_row_stride", "a_stage_elems", "b_stage_elems", "lds_bytes")


def test_ablations_differ_from_the_default_in_one_choice(gemm_lib):
    base = dft.gemm_f32_tile_config(dft.VARIANT_MFMA)
    auto = dft.gemm_f32_tile_config(dft.VARIANT_AUTO)  # AUTO describes its large-problem choice
    big = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_256x256_BK32_PIPE)
    assert auto | {"variant": dft.VARIANT_MFMA_256x256_BK32_PIPE} == big
    assert big["bk"] == 32 and big["direct_to_lds"] == 2
    s1 = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_STAGES1)
    assert s1["stages"] == 1 and s1["barriers_per_tile"] == 2
    assert s1 | {"variant": 1, "stages": 2, "barriers_per_tile": 1, "lds_bytes": base["lds_bytes"]} == base
    plain = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_NOPAD)
    assert all(plain[k] == 0 for k in LAYOUT_KEYS[:8])
    assert plain | {"variant": 1} | {k: base[k] for k in LAYOUT_KEYS} == base
    sc = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_SCALAR)
    assert sc["vec_width"] == 1
    assert sc | {"variant": 1, "vec_width": 4} | {k: base[k] for k in LAYOUT_KEYS} == base
    m16 = dft.gemm_f32_tile_config(dft.VARIANT_MFMA16)
    assert m16["mfma_block"] == 16 and base["mfma_block"] == 32
    direct = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_DIRECT)
    assert direct["direct_to_lds"] == 1 and base["direct_to_lds"] == 0
    assert direct | {"variant": 1, "direct_to_lds": 0} | {k: base[k] for k in LAYOUT_KEYS} == base


def test_auto_variant_selection(gemm_lib):
    av = dft.gemm_f32_auto_variant
    # measured fastest (or within 3 % of it) on one MI355X (256 CUs) for each of these shapes
    assert av(4096, 4096, 4096, 256) == dft.VARIANT_MFMA_256x256_BK32_PIPE  # 256 tiles of 256x256: 1 full round
    assert av(8192, 8192, 8192, 256) == dft.VARIANT_MFMA_256x256_BK32_PIPE
    assert av(4096, 4096, 1024, 256) == dft.VARIANT_MFMA_256x256_BK32_PIPE
    assert av(4096, 2048, 4096, 256) == dft.VARIANT_MFMA_128_BK32_DIRECT  # 512 tiles of 128x128: two per CU
    assert av(8192, 1024, 2048, 256) == dft.VARIANT_MFMA_128_BK32_DIRECT  # 256 tiles of 256x128: one per CU
    assert av(6144, 6144, 2048, 256) == dft.VARIANT_MFMA_128_BK32_DIRECT  # 2304 tiles: 9 full rounds
    assert av(2048, 2048, 4096, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT  # 1024 tiles of 64x64 against 256 of 128x128
    assert av(3000, 3000, 1000, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    assert av(512, 4096, 4096, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT   # 512 tiles of 64x64: 131 against 114 pipelined
    assert av(2048, 256, 16384, 256) == dft.VARIANT_MFMA_32x64_KS4  # deep K, 128 tiles of 64x64: split K
    assert av(1000, 999, 513, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    # ragged grids: edge tiles move back to end at M or N, so only quantisation counts
    assert av(2000, 2000, 1024, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    assert av(5000, 3000, 2000, 256) == dft.VARIANT_MFMA_256x256_BK32_PIPE  # 240 tiles of 256x256
    assert av(6000, 6000, 6000, 256) == dft.VARIANT_MFMA_128_BK32_DIRECT  # 2209 tiles in 9 rounds
    assert av(4095, 4095, 4095, 256) == dft.VARIANT_MFMA_256x256_BK32_PIPE
    assert av(5120, 5120, 5120, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT  # 6400 tiles: 25 full rounds
    # a dimension below the tile: every workgroup of the big kernels is an edge one
    assert av(200, 8192, 4096, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    assert av(4096, 4096, 2048, 4096) == dft.VARIANT_MFMA_64_KS4  # many more CUs than big tiles
    assert av(-1, 4, 4, 256) == dft.GEMM_ERR_INVALID_DIM
    assert av(4, 4, 4, 0) == dft.GEMM_ERR_INVALID_DIM


def test_auto_variant_splits_k_for_few_deep_tiles(gemm_lib):
    av = dft.gemm_f32_auto_variant

    def ax_(M, N, K):  # row alignment as for packed operands (lda = K, ldb = N)
        return dft.gemm_f32_auto_variant_ex(M, N, K, 256, int(K % 4 == 0), int(N % 4 == 0))

    # measured fastest on one MI355X (256 CUs): K split inside the workgroup when few tiles meet a deep K
    assert av(2048, 256, 16384, 256) == dft.VARIANT_MFMA_32x64_KS4   # 101 TF against 54 for 64x64x32
    assert av(1024, 512, 16384, 256) == dft.VARIANT_MFMA_32x64_KS4
    assert av(1024, 1024, 8192, 256) == dft.VARIANT_MFMA_64_KS4      # 256 tiles: 118 against 105
    assert av(4096, 256, 8192, 256) == dft.VARIANT_MFMA_64_KS4
    assert av(512, 512, 16384, 256) == dft.VARIANT_MFMA_32x32_KS8    # 94 against 27
    assert av(256, 256, 65536, 256) == dft.VARIANT_MFMA_32x32_KS8
    # enough tiles, or too short a K: no split
    assert av(512, 4096, 4096, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    assert av(2048, 256, 256, 256) == dft.VARIANT_MFMA_32x64_KS4    # one round of 32x64 tiles: 37 against 33
    assert av(2176, 192, 448, 256) == dft.VARIANT_MFMA_32x64_KS4    # 43 against 33
    assert av(1536, 384, 320, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT  # two rounds of 32x64 tiles: 40 against 29
    assert av(2048, 256, 64, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT   # below one K tile per group
    assert av(1000, 1000, 1000, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT  # 84 against 81 for two groups
    assert av(1000, 1000, 512, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT
    # from K = 1024 when the split's grid has at most one tile per CU
    assert av(512, 512, 1024, 256) == dft.VARIANT_MFMA_32x32_KS8         # 43 against 22
    assert av(1000, 512, 1024, 256) == dft.VARIANT_MFMA_32x64_KS4        # 62 against 42
    assert av(1000, 1000, 2000, 256) == dft.VARIANT_MFMA_64_KS4          # 92 against 87
    # and from K = 512 for the smaller split tiles
    assert av(512, 512, 512, 256) == dft.VARIANT_MFMA_32x32_KS8          # 28 against 17
    assert av(256, 256, 256, 256) == dft.VARIANT_MFMA_32x32_KS8          # 5.3 against 3.7
    assert av(768, 512, 768, 256) == dft.VARIANT_MFMA_32x64_KS4          # 41 against 30
    assert av(2048, 256, 512, 256) == dft.VARIANT_MFMA_32x64_KS4         # 46 against 35
    assert av(1024, 1024, 512, 256) == dft.VARIANT_MFMA_64_BK32_DIRECT   # 82 against 78 for two groups
    assert ax_(1500, 768, 1025) == dft.VARIANT_MFMA_64_BK32_DIRECT         # two rounds: split 44 against 51
    assert ax_(768, 1536, 1025) == dft.VARIANT_MFMA_64_BK32_DIRECT
    # a deep K still splits over several rounds of tiles
    assert av(768, 768, 8192, 256) == dft.VARIANT_MFMA_32x32_KS8         # 68 against 57
    # unaligned operands (odd K: A's rows; odd N: B's), measured per alignment class
    ax = dft.gemm_f32_auto_variant_ex
    assert ax(2048, 256, 16383, 256, 0, 1) == dft.VARIANT_MFMA_32x64_KS4   # 95 against 49
    assert ax(2048, 255, 16384, 256, 1, 0) == dft.VARIANT_MFMA_32x64_KS4   # 79 against 43
    assert ax(1024, 1023, 8192, 256, 1, 0) == dft.VARIANT_MFMA_64_KS4      # 108 against 85
    assert ax(1023, 1023, 8191, 256, 0, 0) == dft.VARIANT_MFMA_64_KS4
    assert ax(512, 511, 16384, 256, 1, 0) == dft.VARIANT_MFMA_32x32_KS8    # 67 against 21


def test_auto_variant_by_operand_alignment(gemm_lib):
    ax = dft.gemm_f32_auto_variant_ex
    # both aligned: the same as gemm_f32_auto_variant
    for shape in [(4096, 4096, 4096), (2048, 2048, 4096), (4096, 2048, 4096), (6000, 6000, 6000)]:
        assert ax(*shape, 256, 1, 1) == dft.gemm_f32_auto_variant(*shape, 256)
    # measured fastest on one MI355X for each alignment class (odd K: A's rows unaligned; odd N: B's)
    assert ax(4096, 4096, 4095, 256, 0, 1) == dft.VARIANT_MFMA_256x256_BK32_PIPE
    assert ax(4096, 4095, 4096, 256, 1, 0) == dft.VARIANT_MFMA_DIRECT   # 4-byte B copies are cheap at 256x128
    assert ax(8192, 8191, 8192, 256, 1, 0) == dft.VARIANT_MFMA_DIRECT
    assert ax(4095, 4095, 4095, 256, 0, 0) == dft.VARIANT_MFMA_256x256_BK32_PIPE
    assert ax(6000, 6000, 5999, 256, 0, 1) == dft.VARIANT_MFMA_128_BK32_DIRECT
    assert ax(4096, 2047, 4096, 256, 1, 0) == dft.VARIANT_MFMA_DIRECT
    assert ax(3000, 2999, 3000, 256, 1, 0) == dft.VARIANT_MFMA_64_KS2   # only B unaligned: 117 against 107
    assert ax(2048, 1023, 2048, 256, 1, 0) == dft.VARIANT_MFMA_64_KS2   # 105 against 92
    assert ax(4096, 2047, 4096, 256, 1, 0) == dft.VARIANT_MFMA_DIRECT   # 125 against 124
    assert ax(1000, 999, 513, 256, 0, 0) == dft.VARIANT_MFMA_64_KS2      # 62 against 53
    assert ax(1000, 999, 513, 256, 1, 1) == dft.VARIANT_MFMA_64_BK32_DIRECT
    assert ax(2047, 2047, 2047, 256, 0, 0) == dft.VARIANT_MFMA_64_BK32_PIPE  # neither aligned, several rounds
    assert ax(1000, 999, 1025, 256, 0, 0) == dft.VARIANT_MFMA_64_KS4      # 71 against 74 (KS2) and 60
    assert ax(2000, 1999, 1025, 256, 0, 0) != dft.VARIANT_MFMA_64_KS2     # multi-round: no two-group split
    assert ax(-1, 4, 4, 256, 1, 1) == dft.GEMM_ERR_INVALID_DIM


# ---- host-side argument validation: every case returns before any device call ----
FAKE_A, FAKE_B, FAKE_C = 0x10000, 0x200000, 0x4000000  # never dereferenced


def call(M, N, K, A=FAKE_A, lda=None, B=FAKE_B, ldb=None, C=FAKE_C, ldc=None, variant=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return dft.gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, None, variant)


@pytest.mark.parametrize("dims", [(-1, 4, 4), (4, -1, 4), (4, 4, -1)])
def test_negative_dims(dims, gemm_lib):
    assert call(*dims) == dft.GEMM_ERR_INVALID_DIM


@pytest.mark.parametrize("kw", [dict(lda=3), dict(ldb=7), dict(ldc=7), dict(lda=0), dict(ldc=-1)])
def test_small_leading_dimension(kw, gemm_lib):
    assert call(5, 8, 4, **kw) == dft.GEMM_ERR_INVALID_LD


def test_leading_dimension_with_zero_extent(gemm_lib):
    # ld must still be >= 1 when the width is 0
    assert call(3, 0, 0, lda=0) == dft.GEMM_ERR_INVALID_LD
    assert call(3, 0, 0) == dft.GEMM_OK  # N == 0: nothing to do


@pytest.mark.parametrize("kw", [dict(A=0), dict(B=0), dict(C=0)])
def test_null_operands(kw, gemm_lib):
    assert call(5, 8, 4, **kw) == dft.GEMM_ERR_NULL


def test_null_allowed_for_empty_extent(gemm_lib):
    assert call(0, 8, 4, A=0, B=0, C=0) == dft.GEMM_OK
    assert call(5, 0, 4, A=0, B=0, C=0) == dft.GEMM_OK


def test_alias(gemm_lib):
    # C overlapping A's last element
    M, N, K = 4, 4, 4
    a_end = FAKE_A + ((M - 1) * K + K) * 4
    assert call(M, N, K, C=a_end - 4) == dft.GEMM_ERR_ALIAS
    assert call(M, N, K, C=FAKE_B) == dft.GEMM_ERR_ALIAS
    assert call(M, N, K, C=FAKE_B - 4) == dft.GEMM_ERR_ALIAS  # C's span reaches into B


def test_too_large(gemm_lib):
    assert call(1 << 40, 4, 1 << 30, lda=1 << 30) == dft.GEMM_ERR_TOO_LARGE


def test_unknown_variant(gemm_lib):
    assert call(4, 4, 4, variant=99) == dft.GEMM_ERR_UNSUPPORTED
    assert call(4, 4, 4, variant=-1) == dft.GEMM_ERR_UNSUPPORTED


def test_binding_requires_the_library(tmp_path):
    with pytest.raises(ImportError):
        dft.library(tmp_path / "missing.so")


# ---- split-K: host-side checks and pure queries ----
def splitk(M, N, K, ws=0x9000000, ws_bytes=1 << 40, splits=2, **kw):
    lda, ldb, ldc = max(K, 1), max(N, 1), max(N, 1)
    return dft.gemm_f32_splitk(M, N, K, kw.get("A", FAKE_A), lda, kw.get("B", FAKE_B), ldb, kw.get("C", FAKE_C), ldc,
                               ws, ws_bytes, splits, None)


def test_splitk_argument_checks(gemm_lib):
    assert splitk(64, 64, 64, splits=-1) == dft.GEMM_ERR_INVALID_DIM
    assert splitk(64, 64, 64, splits=65) == dft.GEMM_ERR_INVALID_DIM
    assert splitk(64, 64, 64, ws=0) == dft.GEMM_ERR_WORKSPACE
    assert splitk(64, 64, 64, ws_bytes=2 * 64 * 64 * 4 - 1) == dft.GEMM_ERR_WORKSPACE
    assert splitk(64, 64, 64, ws=FAKE_C) == dft.GEMM_ERR_ALIAS          # workspace over C
    assert splitk(64, 64, 64, ws=FAKE_A) == dft.GEMM_ERR_ALIAS          # workspace over A
    assert splitk(-1, 64, 64) == dft.GEMM_ERR_INVALID_DIM
    assert splitk(0, 64, 64, ws=0) == dft.GEMM_OK                       # nothing to do
    assert splitk(64, 0, 64, ws=0) == dft.GEMM_OK
    for bad in (-1, dft.VARIANT_COUNT):  # an unknown slice kernel is refused before anything else
        assert dft.gemm_f32_splitk_ex(64, 64, 64, FAKE_A, 64, FAKE_B, 64, FAKE_C, 64, 0, 0, 2, None,
                                      bad) == dft.GEMM_ERR_UNSUPPORTED


def test_splitk_queries(gemm_lib):
    assert dft.gemm_f32_splitk_auto_variant() == dft.VARIANT_MFMA_DIRECT
    # 2048 x 256 x 16384: 16 tiles of 256 x 128 -> 256/16 = 16 slices (<= 1024 K tiles / 8)
    assert dft.gemm_f32_splitk_auto_splits(2048, 256, 16384, 256) == 16
    assert dft.gemm_f32_splitk_workspace_bytes(2048, 256, 16384, 0, 256) == 16 * 2048 * 256 * 4
    assert dft.gemm_f32_splitk_workspace_bytes(2048, 256, 16384, 5, 256) == 5 * 2048 * 256 * 4
    assert dft.gemm_f32_splitk_auto_splits(512, 4096, 4096, 256) == 4      # 64 tiles
    assert dft.gemm_f32_splitk_auto_splits(4096, 4096, 4096, 256) == 1    # 512 tiles: no split
    assert dft.gemm_f32_splitk_workspace_bytes(4096, 4096, 4096, 0, 256) == 0
    assert dft.gemm_f32_splitk_auto_splits(64, 64, 100, 256) == 1         # too few K tiles
    assert dft.gemm_f32_splitk_auto_splits(128, 128, 1 << 20, 256) == 64  # capped at 64
    assert dft.gemm_f32_splitk_auto_splits(-1, 4, 4, 256) == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_f32_splitk_workspace_bytes(4, 4, 4, 99, 256) == dft.GEMM_ERR_INVALID_DIM


def test_every_binding_declares_its_full_signature(gemm_lib):
    """ctypes passes an argument with no declared type as a C int, which
    truncates a 64-bit device pointer; every exported function of both
    libraries must have its argument list declared, with pointers as
    pointer types and as many arguments as the header declares."""
    from dense_fp32_tiled_amd import lds_probe

    probe = lds_probe.load()
    for lib, header in ((gemm_lib, HEADER), (probe, PROBE_HEADER)):
        text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
        for name, params in re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(([^)]*)\)", text, flags=re.M):
            fn = getattr(lib, name)
            assert fn.argtypes is not None, f"{name} has no declared argtypes"
            decl = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
            assert len(fn.argtypes) == len(decl), name
            for d, t in zip(decl, fn.argtypes):
                if "*" in d:
                    assert t is ctypes.c_void_p or t is ctypes.c_char_p or hasattr(t, "contents"), (name, d, t)


# ---- 16-bit inputs (gemm_mixed_f32) ----
@pytest.mark.parametrize("variant", range(dft.MIXED_COUNT))
def test_mixed_tile_config_is_consistent(variant, gemm_lib):
    c = dft.gemm_mixed_tile_config(variant)
    assert c["variant"] == variant and c["elem_bytes"] == 2 and c["direct_to_lds"] == 1
    assert c["a_pad"] == 0 and c["b_pad"] == 0
    assert c["stages"] in (2, 3) if c["k_groups"] == 1 else c["stages"] == 2 * c["k_groups"]
    # LDS tiles in 4-byte words: a row of a 16-bit tile holds two elements per word
    assert (c["a_rows"], 2 * c["a_cols"]) == (c["bm"], c["bk"])
    assert (c["b_rows"], 2 * c["b_cols"]) == (c["bk"], c["bn"])
    assert c["lds_bytes"] == c["stages"] * (c["a_stage_elems"] + c["b_stage_elems"]) * 4 <= 160 * 1024
    assert c["threads"] == (c["bm"] // c["tm"]) * (c["bn"] // c["tn"]) * 64 * c["k_groups"]
    assert c["mfma_block"] == 32


def test_mixed_argument_checks(gemm_lib):
    def mixed(M, N, K, input_type=dft.INPUT_BF16, variant=0, A=FAKE_A, B=FAKE_B, C=FAKE_C, lda=None):
        return dft.gemm_mixed_f32(input_type, M, N, K, A, lda or max(K, 1), B, max(N, 1), C, max(N, 1), None, variant)

    assert mixed(4, 4, 4, input_type=2) == dft.GEMM_ERR_UNSUPPORTED
    assert mixed(4, 4, 4, input_type=-1) == dft.GEMM_ERR_UNSUPPORTED
    assert mixed(4, 4, 4, variant=dft.MIXED_COUNT) == dft.GEMM_ERR_UNSUPPORTED
    assert mixed(-1, 4, 4) == dft.GEMM_ERR_INVALID_DIM
    assert mixed(4, 4, 8, lda=7) == dft.GEMM_ERR_INVALID_LD
    assert mixed(4, 4, 4, A=0) == dft.GEMM_ERR_NULL
    assert mixed(0, 4, 4, A=0, B=0, C=0) == dft.GEMM_OK
    # A spans (M - 1) * lda + K two-byte elements: C just past its end is legal, one element earlier aliases
    M, K = 64, 64
    end_a = FAKE_A + ((M - 1) * K + K) * 2
    assert mixed(M, 8, K, C=end_a) != dft.GEMM_ERR_ALIAS
    assert mixed(M, 8, K, C=end_a - 2) == dft.GEMM_ERR_ALIAS
    with pytest.raises(dft.GemmError):
        dft.gemm_mixed_tile_config(dft.MIXED_COUNT)
    assert gemm_lib.gemm_mixed_tile_config(0, None) == dft.GEMM_ERR_NULL


def test_mixed_auto_variant(gemm_lib):
    av = dft.gemm_mixed_auto_variant
    assert av(8192, 8192, 8192, 256) == dft.MIXED_256x256_BK64  # 1024 tiles of 256x256
    assert av(4096, 4096, 4096, 256) == dft.MIXED_256x256_BK64  # 256 tiles
    assert av(2048, 4096, 4096, 256) == dft.MIXED_128x128_BK64  # 128 tiles of 256x256, 512 of 128x128
    # few 256x256 tiles: the 64x64-tile kernels, with K split inside the workgroup when K is deep
    assert av(2048, 256, 16384, 256) == dft.MIXED_32x64_KS4    # 290 TF against 94 for 128x128
    assert av(1024, 1024, 8192, 256) == dft.MIXED_64x64_KS4    # 398 against 184
    assert av(512, 4096, 4096, 256) == dft.MIXED_64x64_KS2     # 527 against 328
    assert av(512, 512, 16384, 256) == dft.MIXED_32x64_KS4
    assert av(1000, 1000, 1000, 256) == dft.MIXED_64x64       # 142 against 96
    assert av(1536, 1536, 4096, 256) == dft.MIXED_64x64
    assert av(3000, 3000, 3000, 256) == dft.MIXED_256x256_S3     # 144 tiles; K not a multiple of 64
    assert av(8000, 8000, 4000, 256) == dft.MIXED_256x256_S3
    assert av(3072, 3072, 3072, 256) == dft.MIXED_256x256_BK64
    assert av(6000, 6000, 6000, 256) == dft.MIXED_256x256_S3     # 576 tiles vs 2209 of 128x128
    assert av(2048, 2048, 2048, 256) == dft.MIXED_64x64         # 544 against 492
    # from K = 1024 the split runs when its grid has at most one tile per CU
    assert av(512, 512, 2048, 256) == dft.MIXED_32x64_KS4       # 103 against 85
    assert av(1024, 512, 1024, 256) == dft.MIXED_32x64_KS4      # 120 against 108
    assert av(1024, 1024, 3072, 256) == dft.MIXED_64x64_KS4     # 331 against 305
    assert av(1536, 768, 2048, 256) == dft.MIXED_64x64_KS2      # 288 tiles of 64x64: no four-group split
    assert av(512, 512, 512, 256) == dft.MIXED_64x64
    assert av(1024, 1024, 1024, 256) == dft.MIXED_64x64_KS2     # 266 against 240 for 64x64_KS4
    assert av(-1, 4, 4, 256) == dft.GEMM_ERR_INVALID_DIM
