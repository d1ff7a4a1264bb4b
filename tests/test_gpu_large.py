"""Operands past 2**31 elements: every index the kernels form from a row and a
leading dimension must be 64-bit.  A (1,048,600 x 2048) and C (1,048,600 x
2050, ldc 2052) each hold more than 2**31 fp32 elements, so a 32-bit offset
anywhere in the load, copy or store path lands on the wrong row (or faults
past the buffer) for the rows beyond that point.

To keep the inputs cheap to build, row i of A is row i % 64 of a seeded
integer-valued block, so C's row i must equal row i % 64 of the oracle's
product of that block with B, bit for bit (every partial sum is an integer
below 2**24).  Rows on both sides of the 2**31-element boundaries of A and
C, the first and last rows and a seeded sample are compared, and the ld gap
and the row after C must keep their NaN sentinel."""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads

pytestmark = pytest.mark.gpu

M, K, N = 1_048_600, 2048, 2050
LDB, LDC = 2052, 2052
PERIOD = 64
SENTINEL_BITS = np.uint32(0x7FC0DEAD)


def checked_rows() -> np.ndarray:
    a_edge = (1 << 31) // K      # first row of A past 2**31 elements
    c_edge = (1 << 31) // LDC    # first row of C past 2**31 elements
    rng = np.random.default_rng(909)
    rows = np.concatenate([np.arange(0, 80), np.arange(a_edge - 40, a_edge + 24), np.arange(c_edge - 40, c_edge + 40),
                           np.arange(M - 80, M), rng.integers(0, M, 256)])
    return np.unique(rows)


@pytest.fixture(scope="module")
def big(gemm_lib):
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    base, b = workloads.make_operands(PERIOD, N, K, "integer", 4242)
    assert M * K > 1 << 31 and M * LDC > 1 << 31
    cref, _ = oracle.reference(base, b)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(base).to(dev).repeat((M + PERIOD - 1) // PERIOD, 1)[:M]
    assert a.is_contiguous() and a.shape == (M, K)
    bbuf = torch.from_numpy(workloads.embed(b, LDB, np.nan)).to(dev)
    c = torch.empty(((M + 1) * LDC,), dtype=torch.float32, device=dev)
    yield torch, a, bbuf, c, cref
    del a, bbuf, c
    torch.cuda.empty_cache()


def check(torch, c, cref):
    rows = checked_rows()
    full = c.view(M + 1, LDC)
    got = full[torch.from_numpy(rows).to(c.device)].cpu().numpy()
    np.testing.assert_array_equal(got[:, :N].astype(np.float64), cref[rows % PERIOD])
    assert np.all(got[:, N:].view(np.uint32) == SENTINEL_BITS), "a write landed in the ld gap of C"
    tail = full[M].cpu().numpy()
    assert np.all(tail.view(np.uint32) == SENTINEL_BITS), "a write landed past the last row of C"


LARGE_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA, dft.VARIANT_MFMA_128_DIRECT, dft.VARIANT_VALU]


@pytest.mark.parametrize("variant", LARGE_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in LARGE_VARIANTS])
def test_offsets_beyond_2_31_elements(variant, big):
    torch, a, bbuf, c, cref = big
    c.view(torch.int32).fill_(int(SENTINEL_BITS))
    st = dft.gemm_f32_ex(M, N, K, a.data_ptr(), K, bbuf.data_ptr(), LDB, c.data_ptr(), LDC,
                         torch.cuda.current_stream().cuda_stream, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    check(torch, c, cref)


def test_splitk_offsets_beyond_2_31_elements(big):
    """Two slices: the workspace holds 2 * M * N partial sums (over 2**32
    elements) and the reduction indexes all of them."""
    torch, a, bbuf, c, cref = big
    c.view(torch.int32).fill_(int(SENTINEL_BITS))
    need = dft.gemm_f32_splitk_workspace_bytes(M, N, K, 2, 256)
    assert need == 2 * M * N * 4
    ws = torch.empty((need // 4,), dtype=torch.float32, device=c.device)
    st = dft.gemm_f32_splitk_ex(M, N, K, a.data_ptr(), K, bbuf.data_ptr(), LDB, c.data_ptr(), LDC, ws.data_ptr(), need,
                                2, torch.cuda.current_stream().cuda_stream, dft.VARIANT_AUTO)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    del ws
    check(torch, c, cref)


# Leading dimensions so wide that a tile's byte span exceeds 31 bits: the
# direct copies address a tile as a uniform base plus a 32-bit per-lane byte
# offset, so such launches must load every tile through registers instead.
# A: 8,388,612 floats per row (>= 2**31 bytes for any tile of 64 rows);
# B: 33,554,436 floats per row (>= 2**31 bytes for a 16-row K tile).
WIDE_LDA = (1 << 23) + 4
WIDE_LDB = (1 << 25) + 4
WIDE_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA_128_BK32_DIRECT,
                 dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_256x256_DIRECT, dft.VARIANT_MFMA_256x256_PIPE,
                 dft.VARIANT_MFMA16_256x256_W4_BK32_PIPE, dft.VARIANT_MFMA_64_BK32_DIRECT]


@pytest.fixture(scope="module")
def torch_dev(gemm_lib):
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def wide_operands(torch, a, b, lda, ldb, dtype=None):
    """Device copies of a and b embedded with leading dimensions lda / ldb
    (NaN in the gaps), built on the device to keep host memory small."""
    (M, K), N = a.shape, b.shape[1]
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    if dtype is not None:
        ta, tb = ta.to(dtype), tb.to(dtype)
    abuf = torch.full((M * lda,), float("nan"), device="cuda", dtype=ta.dtype)
    bbuf = torch.full((K * ldb,), float("nan"), device="cuda", dtype=tb.dtype)
    abuf.view(M, lda)[:, :K] = ta
    bbuf.view(K, ldb)[:, :N] = tb
    return abuf, bbuf


@pytest.mark.parametrize("variant", WIDE_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in WIDE_VARIANTS])
@pytest.mark.parametrize("wide", ["a", "b"])
def test_wide_leading_dimension_falls_back_to_registers(wide, variant, torch_dev):
    torch = torch_dev
    M, N, K = 300, 260, 100  # the first 256 x 256 (and smaller) tiles are interior
    a, b = workloads.make_operands(M, N, K, "integer", 515)
    cref, _ = oracle.reference(a, b)
    lda, ldb = (WIDE_LDA, N) if wide == "a" else (K, WIDE_LDB)
    abuf, bbuf = wide_operands(torch, a, b, lda, ldb)
    c = torch.full((M, N), float("nan"), device="cuda")
    st = dft.gemm_f32_ex(M, N, K, abuf.data_ptr(), lda, bbuf.data_ptr(), ldb, c.data_ptr(), N,
                         torch.cuda.current_stream().cuda_stream, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), cref)
    del abuf, bbuf
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wide", ["a", "b"])
def test_wide_leading_dimension_bf16(wide, torch_dev):
    torch = torch_dev
    M, N, K = 300, 260, 136
    a, b = workloads.make_operands(M, N, K, "integer", 516)
    (abits, af), (bbits, bf) = workloads.to_16bit(a, "bf16"), workloads.to_16bit(b, "bf16")
    cref, _ = oracle.reference(af, bf)
    lda, ldb = (WIDE_LDA, N) if wide == "a" else (K, WIDE_LDB)
    abuf, bbuf = wide_operands(torch, af, bf, lda, ldb, dtype=torch.bfloat16)
    c = torch.full((M, N), float("nan"), device="cuda")
    st = dft.gemm_mixed_f32(dft.INPUT_BF16, M, N, K, abuf.data_ptr(), lda, bbuf.data_ptr(), ldb, c.data_ptr(), N,
                            torch.cuda.current_stream().cuda_stream, dft.MIXED_AUTO)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c.cpu().numpy().astype(np.float64), cref)
    del abuf, bbuf
    torch.cuda.empty_cache()
