"""Seeded synthetic inputs for the masked, tiled fp32 matrix multiply.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no matrix-multiply arithmetic: it only draws operands and
places them in (possibly padded) row-major buffers.

Workload shapes follow the tiled matmul the pages build ("My Triton From
Scratch, Part 14: Shared-Memory Tiles", section "The canonical source pattern":
A is M x K, B is K x N, both row-major, C = A @ B).  Five shapes are used:

  name        M      N      K      entries
  small128    128    128    128    uniform[-1, 1)      one tile, several K tiles
  ragged      1000   999    513    uniform[-1, 1)      every tile edge masked
  square4096  4096   4096   4096   standard normal     compute-bound square
  deepk       2048   256    16384  uniform[-1, 1)      long K loop
  square8192  8192   8192   8192   standard normal     large square

plus one extra shape, shard8_4096 (512 x 4096 x 4096, standard normal): the
rows of square4096 that one of eight GPUs would own.

Generator: NumPy PCG64 (``numpy.random.default_rng(seed)``); A is drawn before
B from one generator.  Uniform entries are ``uniform(-1, 1)`` cast to float32;
normal entries are ``standard_normal(dtype=float32)``.  "Integer" operands
(entries uniform in {-4, ..., 4}) make every partial sum of a product exactly
representable in fp32, so any summation order gives the same bits.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class GemmConfig:
    name: str
    M: int
    N: int
    K: int
    dist: str  # "uniform" or "normal"
    seed: int
    sampled: bool  # large shapes: the oracle checks sampled rows and columns

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def min_bytes(self) -> int:
        return 4 * (self.M * self.K + self.K * self.N + self.M * self.N)


CONFIGS: tuple[GemmConfig, ...] = (
    GemmConfig("small128", 128, 128, 128, "uniform", 1, False),
    GemmConfig("ragged", 1000, 999, 513, "uniform", 2, False),
    GemmConfig("square4096", 4096, 4096, 4096, "normal", 3, True),
    GemmConfig("deepk", 2048, 256, 16384, "uniform", 4, False),
    GemmConfig("square8192", 8192, 8192, 8192, "normal", 5, True),
)

# One GPU's share of square4096 when its rows are split over eight GPUs (the
# row-block sharding of C = A @ B): too few 256 x 128 output tiles to fill
# the chip, so it exercises the smaller-tile kernels.
EXTRA_CONFIGS: tuple[GemmConfig, ...] = (
    GemmConfig("shard8_4096", 512, 4096, 4096, "normal", 6, False),
)

CONFIG_BY_NAME = {c.name: c for c in CONFIGS + EXTRA_CONFIGS}

# Seed offsets: sampled rows/columns use seed + 100, integer operands seed + 200.
SAMPLE_SEED_OFFSET = 100
INTEGER_SEED_OFFSET = 200


def draw(rng: np.random.Generator, shape: tuple[int, int], dist: str) -> np.ndarray:
    """One float32 matrix of the given distribution."""
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(size=shape, dtype=np.float32)
    if dist == "integer":
        return rng.integers(-4, 5, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_operands(M: int, N: int, K: int, dist: str, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Packed row-major A (M x K) and B (K x N), A drawn first."""
    rng = np.random.default_rng(seed)
    a = draw(rng, (M, K), dist)
    b = draw(rng, (K, N), dist)
    return a, b


def config_operands(cfg: GemmConfig, integer: bool = False) -> tuple[np.ndarray, np.ndarray]:
    if integer:
        return make_operands(cfg.M, cfg.N, cfg.K, "integer", cfg.seed + INTEGER_SEED_OFFSET)
    return make_operands(cfg.M, cfg.N, cfg.K, cfg.dist, cfg.seed)


# ---- 16-bit inputs (the mixed-precision kernels) ----------------------------
# Operands are drawn as above in float32 and then stored in a 16-bit format:
# the GEMM's inputs ARE the 16-bit values, and their exact float32 values (a
# widening, which loses nothing) are what the oracle multiplies.

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, rounded to nearest, ties to
    even (the upper 16 bits of the float32 pattern after adding half a unit
    of the dropped part, plus one more when the kept part is odd).  Inputs
    here are finite."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = bits + 0x7FFF + ((bits >> 16) & 1)
    return (rounded >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_16bit(x: np.ndarray, input_type: str) -> tuple[np.ndarray, np.ndarray]:
    """(16-bit patterns, their exact float32 values) of float32 operands, for
    input_type "bf16" or "f16" (IEEE binary16, round to nearest even)."""
    if input_type == "bf16":
        bits = to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    if input_type == "f16":
        h = np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
        return h.view(np.uint16), h.astype(np.float32)
    raise ValueError(f"unknown 16-bit input type {input_type!r}")


def sample_indices(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct indices in [0, n): always 0 and n-1, the rest drawn
    without replacement from a seeded generator."""
    if n <= count:
        return np.arange(n, dtype=np.int64)
    rng = np.random.default_rng(seed)
    inner = rng.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    idx = np.concatenate([[0, n - 1], inner]).astype(np.int64)
    return np.sort(idx)


def sample_rows_cols(cfg: GemmConfig, count: int = 64) -> tuple[np.ndarray, np.ndarray]:
    seed = cfg.seed + SAMPLE_SEED_OFFSET
    return sample_indices(cfg.M, count, seed), sample_indices(cfg.N, count, seed + 1)


def embed(mat: np.ndarray, ld: int, fill: float = float("nan"), extra_rows: int = 0) -> np.ndarray:
    """Place a rows x cols matrix in a row-major buffer of leading dimension
    ``ld`` (>= cols).  Gap columns and ``extra_rows`` trailing rows hold
    ``fill``.  Returns the flat buffer; element (r, c) is at r * ld + c."""
    rows, cols = mat.shape
    assert ld >= cols
    buf = np.full((rows + extra_rows) * ld, fill, dtype=np.float32)
    view = buf[: rows * ld].reshape(rows, ld)
    view[:, :cols] = mat
    return buf
