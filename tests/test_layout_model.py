"""The LDS layout and bank model in the GPU library's host code, against the
values the pages print (tests/golden/layout_pins.json).  CPU only."""

from __future__ import annotations

import json
from pathlib import Path

import pytest

import dense_fp32_tiled_amd as dft

PINS = json.loads((Path(__file__).resolve().parent / "golden" / "layout_pins.json").read_text())


def test_bank_maps(gemm_lib):
    p = PINS["bank_maps"]
    for stride, key in ((16, "stride16"), (17, "stride17")):
        banks = [dft.gemm_lds_bank(dft.gemm_lds_offset(4, 16, stride - 16, 1, 0, r, p["column"]), p["banks"])
                 for r in p["rows"]]
        assert banks == p[key]


def test_page_pad_rule(gemm_lib):
    for columns, rows, pad in PINS["page_pad"]["cases"]:
        assert dft.gemm_lds_page_pad(columns, rows, PINS["page_pad"]["banks"]) == pad


def test_declaration_sizes(gemm_lib):
    for rows, cols, size in PINS["declarations"]["cases"]:
        st, stride, stage, total, nbytes = dft.gemm_lds_layout(rows, cols, 0, 1)
        assert st == 0 and stride == cols and stage == size and total == size and nbytes == 4 * size


def test_padded_two_stage_layout(gemm_lib):
    p = PINS["padded_two_stage"]
    st, stride, stage, total, nbytes = dft.gemm_lds_layout(p["rows"], p["cols"], p["pad"], p["stages"])
    assert (st, stride, stage, total, nbytes) == (0, p["row_stride"], p["stage_elems"], p["total_elems"], p["bytes"])
    for s, r, c, off in p["offsets"]:
        assert dft.gemm_lds_offset(p["rows"], p["cols"], p["pad"], p["stages"], s, r, c) == off


def test_layout_rejects_invalid(gemm_lib):
    assert dft.gemm_lds_layout(0, 16, 0, 1)[0] == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_lds_layout(4, 16, -1, 1)[0] == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_lds_layout(4, 16, 0, 0)[0] == dft.GEMM_ERR_INVALID_DIM
    for coords in [(2, 0, 0), (0, 4, 0), (0, 0, 16), (-1, 0, 0), (0, -1, 0), (0, 0, -1)]:
        assert dft.gemm_lds_offset(4, 16, 1, 2, *coords) == -1
    assert dft.gemm_lds_bank(-1, 32) == -1 and dft.gemm_lds_bank(5, 0) == -1
    assert dft.gemm_lds_page_pad(0, 4, 32) == -1


def test_offsets_are_a_bijection_onto_the_padded_layout(gemm_lib):
    rows, cols, pad, stages = 5, 7, 3, 2
    _, stride, stage_elems, total, _ = dft.gemm_lds_layout(rows, cols, pad, stages)
    seen = set()
    for s in range(stages):
        for r in range(rows):
            for c in range(cols):
                off = dft.gemm_lds_offset(rows, cols, pad, stages, s, r, c)
                assert 0 <= off < total and off % stride < cols  # never lands in padding
                seen.add(off)
    assert len(seen) == stages * rows * cols


def test_conflict_degree_matches_page_example(gemm_lib):
    # four rows of the A tile read the same column at once, one warp of 32 lanes
    for stride, degree in ((16, 2), (17, 1)):
        words = [r * stride for r in range(4)]
        assert dft.gemm_lds_conflict_degree(words, 1, 32, 32) == degree


def test_conflict_degree_rules(gemm_lib):
    cd = dft.gemm_lds_conflict_degree
    assert cd([0] * 64, 1, 64, 64) == 1                       # broadcast of one address
    assert cd(list(range(64)), 1, 64, 64) == 1                # consecutive words
    assert cd([64 * l for l in range(64)], 1, 64, 64) == 64   # all in bank 0
    assert cd([64 * l for l in range(64)], 1, 64, 1) == 1     # one lane per service group
    assert cd([2 * l for l in range(64)], 1, 64, 64) == 2     # stride 2 over 64 banks
    assert cd([2 * l for l in range(64)], 1, 32, 32) == 2
    assert cd([4 * l for l in range(16)], 4, 64, 16) == 1     # 16 x 16 B covers 64 banks once
    assert cd([8 * l for l in range(16)], 4, 64, 16) == 2
    assert cd([], 1, 64, 64) == -1


@pytest.mark.parametrize("variant", [dft.VARIANT_MFMA, dft.VARIANT_VALU])
def test_chosen_pads_are_conflict_free_for_the_fragment_reads(variant, gemm_lib):
    """The pads the kernels are compiled with make their hot LDS reads
    conflict-free under the library's own bank geometry."""
    c = dft.gemm_f32_tile_config(variant)
    g128 = (c["lds_banks_b128"], c["lds_lanes_b128"])
    g32 = (c["lds_banks_b32"], c["lds_lanes_b32"])
    if variant == dft.VARIANT_MFMA:
        kh = c["bk"] // 2
        a = [(l % 32) * c["a_row_stride"] + (l // 32) * kh for l in range(64)]
        b = [(l // 32) * kh * c["b_row_stride"] + (l % 32) for l in range(64)]
        assert dft.gemm_lds_conflict_degree(a, 4, *g128) == 1
        assert dft.gemm_lds_conflict_degree(b, 1, *g32) == 1
        nopad = dft.gemm_f32_tile_config(dft.VARIANT_MFMA_NOPAD)
        a0 = [(l % 32) * nopad["a_row_stride"] + (l // 32) * kh for l in range(64)]
        assert dft.gemm_lds_conflict_degree(a0, 4, *g128) == 4  # rows 0, 4, 8, 12 share banks
    else:
        tn = c["bn"] // c["tn"]
        a = [(l // tn) * 4 for l in range(64)]
        b = [(l % tn) * 4 for l in range(64)]
        assert dft.gemm_lds_conflict_degree(a, 4, *g128) == 1
        assert dft.gemm_lds_conflict_degree(b, 4, *g128) == 1


def test_geometry_is_the_measured_one(gemm_lib):
    """The pads are derived for the geometry the LDS probe measured on gfx950:
    4-byte accesses 32 banks x 32 lanes per pass, 16-byte accesses 64 banks x
    16 lanes per pass."""
    c = dft.gemm_f32_tile_config(dft.VARIANT_MFMA)
    assert (c["lds_banks_b32"], c["lds_lanes_b32"], c["lds_banks_b128"], c["lds_lanes_b128"]) == (32, 32, 64, 16)
