"""Properties of the compiled kernels read from their gfx950 assembly
(hipcc -S on the library's device code).  CPU only: the code is
cross-compiled for gfx950 here.

* The VALU inner product is fully unrolled: one basic block holds all
  BK x TM x TN = 16 x 8 x 8 fused multiply-adds of a K tile (the pages'
  "Unrolling the inner dot loop", whose loop-control overhead this removes).
* The default MFMA kernel's K tile is straight-line code: every MFMA of a
  tile but the last step's (which runs after the barrier) sits in one block.
* No packed fp32 instruction (v_pk_fma_f32, v_pk_mul_f32, v_pk_add_f32) is
  emitted anywhere: the build disables them.
* In the bf16 default kernel's K loop the LDS fragment reads for the next
  step alternate one for one with the current step's MFMAs instead of
  issuing in a burst ahead of them."""

from __future__ import annotations

import re

import pytest

from dense_fp32_tiled_amd import build


@pytest.fixture(scope="module")
def functions():
    text = build.device_assembly()
    labels = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", text, re.M)]
    out = {}
    for k, (pos, name) in enumerate(labels):
        end = labels[k + 1][0] if k + 1 < len(labels) else len(text)
        out[name] = text[pos:end]
    return text, out


def max_per_block(body: str, pattern: str) -> int:
    blocks = re.split(r"^\.LBB\d+_\d+:", body, flags=re.M)
    return max(len(re.findall(pattern, b, re.M)) for b in blocks)


def test_valu_inner_product_is_fully_unrolled(functions):
    _, funcs = functions
    valu = {n: b for n, b in funcs.items() if "gemm_valu_kernel" in n}
    assert len(valu) == 2  # 16-byte and 4-byte load paths
    for name, body in valu.items():
        assert max_per_block(body, r"^\s+v_(?:fmac|fma)_f32") == 16 * 8 * 8, name


def test_default_mfma_tile_is_straight_line(functions):
    _, funcs = functions
    # 256x256x32, 8 waves of 128x64: 4 x 2 blocks x 16 steps = 128 MFMAs per K tile
    default = [b for n, b in funcs.items()
               if "MfmaCfgILi256ELi256ELi32ELi128ELi64ELi2ELi32E" in n and "EEELi4ELi1ELi1ELb1ELi0ELi0EE" in n]
    assert len(default) == 1
    assert max_per_block(default[0], r"^\s+v_mfma_f32_32x32x2_f32") >= 128 - 8


def test_no_packed_fp32_instructions(functions):
    text, _ = functions
    assert not re.search(r"v_pk_(?:fma|mul|add)_f32", text)


def test_m0_is_used_only_by_the_direct_copies(functions):
    """The copy statements write M0 without saving it (they declare it
    clobbered, and the compiler does not preserve a reserved register across
    inline asm).  That is safe only while no compiler-generated code keeps a
    value in M0: every instruction that names m0 must be one of the copies'
    own s_mov_b32 m0 from a scalar register, followed by the wait state and the copy."""
    text, _ = functions
    lines = [l.strip() for l in text.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
    uses = [i for i, l in enumerate(code) if re.search(r"\bm0\b", l)]
    assert uses
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", code[i]), code[i]
        assert code[i + 1] == "s_nop 0", code[i + 1]
        assert code[i + 2].startswith(("global_load_lds_dwordx4 ", "global_load_lds_dword ")), code[i + 2]


def test_bf16_default_loop_alternates_mfmas_and_lds_reads(functions):
    _, funcs = functions
    # 256x256x64 tile, 8 waves of 128x64 (4 x 2 MFMA blocks of 32x32x16), 16-byte copies, 2 stages,
    # pipelined across K tiles: one block holds steps 0..2 of a tile, 8 MFMAs and 8 reads each, and
    # another the last step, after the barrier
    default = [b for n, b in funcs.items() if "gemm_mixed_kernel" in n and
               "MixedCfgILi0ELi256ELi256ELi64ELi128ELi64ELi32E" in n and n.endswith("ELi8ELi2ELi2ELi2EEEEEvlllPKtlS7_lPflll")]
    assert len(default) == 1
    blocks = re.split(r"^\.LBB\d+_\d+:", default[0], flags=re.M)

    def order(block):
        kinds = []
        for line in block.splitlines():
            op = line.strip()
            if op.startswith("v_mfma"):
                kinds.append("M")
            elif op.startswith("ds_read"):
                kinds.append("R")
        return "".join(kinds)

    orders = list(map(order, blocks))
    loop = [o for o in orders if o.count("M") == 24 and "R" in o]
    assert len(loop) == 1
    assert loop[0] == "MR" * 24
    # the last step of a tile, after the barrier, with step 0 of the next tile's reads
    assert "MR" * 8 in orders
