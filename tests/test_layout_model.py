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


def lds_word(cfg, tile, row, col):
    """Word offset (stage 0) of logical (row, col) in a variant's LDS tile."""
    unit, shift, mask = cfg[f"{tile}_swz_unit"], cfg[f"{tile}_swz_shift"], cfg[f"{tile}_swz_mask"]
    phys = col ^ (unit * ((row >> shift) & mask)) if unit else col
    return row * cfg[f"{tile}_row_stride"] + phys


def mfma_accesses(c):
    """Every LDS access of one K tile of an MFMA variant, per wavefront:
    (width in dwords, 64 lane word addresses, whether it is a store)."""
    mb = c["mfma_block"]
    kg = c["bk"] // (64 // mb)
    waves_n = c["bn"] // c["tn"]
    vec = c["vec_width"]
    out = []
    for w in range(c["threads"] // 64):
        wm0, wn0 = (w // waves_n) * c["tm"], (w % waves_n) * c["tn"]
        for mi in range(c["tm"] // mb):
            for q in range(kg // 4):
                out.append((4, [lds_word(c, "a", wm0 + mi * mb + l % mb, (l // mb) * kg + 4 * q) for l in range(64)],
                            False))
        for j in range(kg):  # B reads of block columns 2p, 2p+1 are one ds_read2_b32
            for ni in range(0, c["tn"] // mb, 2):
                pair = [[lds_word(c, "b", (l // mb) * kg + j, wn0 + (ni + e) * mb + l % mb) for e in (0, 1)]
                        for l in range(64)]
                out.append((-2, pair, False))
        for tile, rows, cols in (("a", c["bm"], c["bk"]), ("b", c["bk"], c["bn"])):
            if c["direct_to_lds"]:  # direct copies write 1 KiB of consecutive words: no LDS store instruction
                continue
            vcols = cols // vec
            for i in range(rows * vcols // c["threads"]):
                idx = [w * 64 + l + i * c["threads"] for l in range(64)]
                out.append((vec, [lds_word(c, tile, x // vcols, (x % vcols) * vec) for x in idx], True))
    return out


def degree(c, width, words):
    if width == -2:  # two-address access: served as two 4-byte accesses (measured)
        return max(degree(c, 1, [pair[e] for pair in words]) for e in (0, 1))
    banks = c["lds_banks_b32"] if width == 1 else c["lds_banks_b128"]
    lanes = c["lds_lanes_b32"] if width == 1 else c["lds_lanes_b128"]
    return dft.gemm_lds_conflict_degree(words, width, banks, lanes)


MFMA_LAYOUT_VARIANTS = [dft.VARIANT_MFMA, dft.VARIANT_MFMA16, dft.VARIANT_MFMA_128, dft.VARIANT_MFMA_128_BK32,
                        dft.VARIANT_MFMA_SCALAR, dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA_64_DIRECT,
                        dft.VARIANT_MFMA_256x256_DIRECT, dft.VARIANT_MFMA_256x256_W4_DIRECT,
                        dft.VARIANT_MFMA_256x256_PIPE, dft.VARIANT_MFMA_256x256_BK32_PIPE,
    dft.VARIANT_MFMA16_256x256_DIRECT, dft.VARIANT_MFMA16_256x256_W4_BK32_PIPE, dft.VARIANT_MFMA_64_BK32_DIRECT]


def model_cycles(width, words, store=False):
    """LDS cycles of one access under the search's model (gemm_lds_access_cycles)."""
    if width == -2:  # two-address read of block columns 2p, 2p+1 (NB words apart)
        first = [pair[0] for pair in words]
        return dft.gemm_lds_access_cycles(first, -(words[0][1] - words[0][0]))
    return dft.gemm_lds_access_cycles(words, width + (100 if store else 0))


def free_cycles(width, store=False):
    """Cycles of the same access without a conflict: one per pass."""
    lanes = {(1, False): 32, (4, False): 16, (1, True): 32, (4, True): 8}
    if width == -2:
        return 2 * (64 // 32)
    return 64 // lanes[(width, store)]


# The four-wave 16x16x4 kernel's pipelined fragment addressing (a per-lane
# base plus compile-time offsets) admits no layout whose A-fragment reads are
# conflict-free: the model charges them twice the conflict-free cycles, and
# the probe times them so (8 cycles against 4).
MODEL_DOUBLE_A_READ = {dft.VARIANT_MFMA16_256x256_W4_BK32_PIPE}


@pytest.mark.parametrize("variant", MFMA_LAYOUT_VARIANTS)
def test_mfma_layouts_cost_what_the_model_allows(variant, gemm_lib):
    """Every fragment read and store of the chosen layouts costs the model's
    conflict-free cycles (stores under the measured store geometry), but the
    A reads of the four-wave 16x16x4 kernel (exactly twice); the plain layout
    costs more."""
    c = dft.gemm_f32_tile_config(variant)
    for w, words, store in mfma_accesses(c):
        expect = free_cycles(w, store)
        if variant in MODEL_DOUBLE_A_READ and w == 4 and not store:
            expect *= 2
        assert model_cycles(w, words, store) == expect, (w, store)
    plain = c | {k: 0 for k in ("a_pad", "a_swz_unit", "b_pad", "b_swz_unit")}
    plain["a_row_stride"], plain["b_row_stride"] = c["a_cols"], c["b_cols"]
    cost = sum(model_cycles(w, words, st) for w, words, st in mfma_accesses(c))
    assert sum(model_cycles(w, words, st) for w, words, st in mfma_accesses(plain)) > cost


@pytest.mark.parametrize("variant", MFMA_LAYOUT_VARIANTS)
def test_built_layouts_match_the_search(variant, gemm_lib):
    """The layouts compiled into the kernels (generated at build time) are the
    ones the exported search returns for the same shape."""
    c = dft.gemm_f32_tile_config(variant)
    st, la, lb = dft.gemm_lds_choose_mfma_layout(c["bm"], c["bn"], c["bk"], c["tm"], c["tn"], c["mfma_block"],
                                                 c["vec_width"], c["direct_to_lds"])
    assert st == 0
    assert la == (c["a_pad"], c["a_swz_unit"], c["a_swz_shift"], c["a_swz_mask"])
    assert lb == (c["b_pad"], c["b_swz_unit"], c["b_swz_shift"], c["b_swz_mask"])


def test_direct_copy_layouts_are_unpadded(gemm_lib):
    """With direct copies the search may only swizzle: a copy instruction
    fills consecutive LDS words, which leaves no room for row padding."""
    for shape in ((256, 128, 16, 64, 64, 32), (128, 128, 16, 64, 64, 32), (256, 128, 16, 64, 64, 16),
                  (128, 128, 32, 64, 64, 32)):
        st, la, lb = dft.gemm_lds_choose_mfma_layout(*shape, 4, 1)
        assert st == 0 and la[0] == 0 and lb[0] == 0
    # 16x16x4 blocks: the search through registers pads B, the direct one cannot
    assert dft.gemm_lds_choose_mfma_layout(256, 128, 16, 64, 64, 16, 4, 0)[2][0] == 4
    assert dft.gemm_lds_choose_mfma_layout(256, 128, 16, 64, 64, 32, 1, 1)[0] == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_lds_choose_mfma_layout(256, 128, 16, 64, 64, 32, 4, 3)[0] == dft.GEMM_ERR_INVALID_DIM


def test_layout_search_rejects_bad_shapes(gemm_lib):
    assert dft.gemm_lds_choose_mfma_layout(256, 128, 16, 64, 64, 8, 4)[0] == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_lds_choose_mfma_layout(256, 128, 6, 64, 64, 32, 4)[0] == dft.GEMM_ERR_INVALID_DIM
    assert dft.gemm_lds_choose_mfma_layout(100, 128, 16, 64, 64, 32, 4)[0] == dft.GEMM_ERR_INVALID_DIM


def test_valu_reads_are_conflict_free(gemm_lib):
    c = dft.gemm_f32_tile_config(dft.VARIANT_VALU)
    tn = c["bn"] // c["tn"]
    a = [(l // tn) * 4 for l in range(64)]
    b = [(l % tn) * 4 for l in range(64)]
    assert degree(c, 4, a) == 1 and degree(c, 4, b) == 1


def test_geometry_is_the_measured_one(gemm_lib):
    """The layouts are derived for the geometry the LDS probe measured on
    gfx950: 4-byte reads 32 banks x 32 lanes per pass, 16-byte reads 64 banks
    x 16 lanes, 16-byte stores 32 banks x 8 lanes."""
    c = dft.gemm_f32_tile_config(dft.VARIANT_MFMA)
    assert (c["lds_banks_b32"], c["lds_lanes_b32"], c["lds_banks_b128"], c["lds_lanes_b128"]) == (32, 32, 64, 16)
    assert dft.gemm_lds_access_cycles([4 * l for l in range(64)], 4) == 4       # 4 conflict-free passes
    assert dft.gemm_lds_access_cycles([4 * l for l in range(64)], 104) == 8     # stores: 8 lanes per pass
    assert dft.gemm_lds_access_cycles([8 * l for l in range(64)], 104) == 16    # 2-way over 32 banks
    assert dft.gemm_lds_access_cycles([8 * l for l in range(64)], 4) == 8       # 2-way over 64 banks
    assert dft.gemm_lds_access_cycles([l for l in range(64)], 1) == 2
    assert dft.gemm_lds_access_cycles([0] * 64, 7) == -1
