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
