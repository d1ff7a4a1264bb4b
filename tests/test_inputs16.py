"""The 16-bit input preparation of the mixed-precision tests (workloads):
rounding fp32 to bfloat16 / binary16 and widening back.  CPU only.

The GEMM's inputs are the 16-bit values themselves; the oracle multiplies
their exact float32 widenings, so these functions must be right for the
parity tests to mean anything.  Pinned against hand-worked bit patterns,
the tie-to-even rule, and torch's own CPU conversions."""

from __future__ import annotations

import numpy as np
import torch

import workloads


def bf16(x):
    return [int(v) for v in workloads.to_bf16_bits(np.array(x, dtype=np.float32))]


def test_bf16_hand_values():
    assert bf16([1.0, -2.5, 0.0, 3.0]) == [0x3F80, 0xC020, 0x0000, 0x4040]
    # 1/3 = 0x3EAAAAAB: the dropped half 0xAAAB is above one half, round up
    assert bf16([1 / 3]) == [0x3EAB]


def test_bf16_ties_go_to_even():
    pats = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0xBF808000], dtype=np.uint32)
    got = [int(v) for v in workloads.to_bf16_bits(pats.view(np.float32))]
    assert got == [0x3F80, 0x3F82, 0x3F80, 0x3F81, 0xBF80]


def test_bf16_agrees_with_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000, dtype=np.float32),
                        rng.uniform(-1, 1, 20000).astype(np.float32) * np.float32(2.0) ** rng.integers(-30, 30, 20000)])
    x = x.astype(np.float32)
    mine = workloads.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(workloads.bf16_bits_to_f32(mine), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_widening_is_exact_and_idempotent():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(5000, dtype=np.float32)
    for kind in ("bf16", "f16"):
        bits, f = workloads.to_16bit(x, kind)
        bits2, f2 = workloads.to_16bit(f, kind)  # a representable value rounds to itself
        assert np.array_equal(bits, bits2) and np.array_equal(f, f2)
        assert np.all(np.abs(f - x) <= np.abs(x) * (2.0 ** -8 if kind == "bf16" else 2.0 ** -11))


def test_f16_agrees_with_torch():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(20000, dtype=np.float32) * 100).astype(np.float32)
    bits, f = workloads.to_16bit(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(f, ref.to(torch.float32).numpy())


def test_integer_operands_are_exact_in_16_bits():
    a, _ = workloads.make_operands(16, 16, 16, "integer", 3)
    for kind in ("bf16", "f16"):
        assert np.array_equal(workloads.to_16bit(a, kind)[1], a)
