"""gemm_f32_splitk_noalloc: split-K whose partial products live in the
library's static per-device array instead of a caller's workspace.  Called
through the C ABI and compared with gemm_f32_splitk (caller's workspace) on
the same inputs and split count: the same kernels in the same order, so the
results must agree bit for bit, and both must meet the oracle's bar.  Two
calls in a row, the second on a smaller problem, so that the array still
holds the first call's (larger) partial products when the second runs."""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5
SENTINEL_BITS = np.uint32(0x7FC0DEAD)
SCRATCH_BYTES = 64 << 20


@pytest.fixture(scope="module")
def torch_gpu(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    return torch


def _device(torch, a, b, ldc):
    M, N = a.shape[0], b.shape[1]
    da = torch.from_numpy(a).cuda()
    db = torch.from_numpy(b).cuda()
    dc = torch.from_numpy(np.full((M + 1) * ldc, SENTINEL_BITS, np.uint32).view(np.float32)).cuda()
    return da, db, dc


def _result(torch, dc, M, N, ldc):
    torch.cuda.synchronize()
    full = dc.cpu().numpy().reshape(M + 1, ldc)
    outside = np.ones(full.shape, bool)
    outside[:M, :N] = False
    assert np.all(full.view(np.uint32)[outside] == SENTINEL_BITS), "a write landed outside the M x N region"
    return full[:M, :N].copy()


def noalloc(torch, a, b, splits, ldc):
    M, K = a.shape
    N = b.shape[1]
    da, db, dc = _device(torch, a, b, ldc)
    st = dft.gemm_f32_splitk_noalloc(M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), ldc, splits,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    return _result(torch, dc, M, N, ldc)


def with_workspace(torch, a, b, splits, ldc):
    M, K = a.shape
    N = b.shape[1]
    da, db, dc = _device(torch, a, b, ldc)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = dft.gemm_f32_splitk_workspace_bytes(M, N, K, splits, cus)
    ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
    st = dft.gemm_f32_splitk(M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), ldc, ws.data_ptr(), need,
                             splits, torch.cuda.current_stream().cuda_stream)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    return _result(torch, dc, M, N, ldc)


# First call large (the deep-K workload, 16 slices of 2048 x 256 = 32 MiB of
# partial products), second smaller; each with explicit and automatic splits.
CALLS = [((2048, 256, 16384), 16), ((300, 200, 3000), 5)]


@pytest.mark.parametrize("auto", [False, True], ids=["explicit", "auto"])
def test_noalloc_matches_workspace_entry_point(auto, torch_gpu):
    torch = torch_gpu
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for (M, N, K), splits in CALLS:
        print(f"noalloc {M}x{N}x{K} splits {0 if auto else splits}", flush=True)
        s = 0 if auto else splits
        if auto:
            assert dft.gemm_f32_splitk_auto_splits(M, N, K, cus) * M * N * 4 <= SCRATCH_BYTES
        for dist in ("integer", "uniform"):
            a, b = workloads.make_operands(M, N, K, dist, 3100 + M + K)
            c_na = noalloc(torch, a, b, s, N + 3)
            c_ws = with_workspace(torch, a, b, s, N + 3)
            assert np.array_equal(c_na.view(np.uint32), c_ws.view(np.uint32)), (M, N, K, dist)
            cref, den = oracle.reference(a, b)
            if dist == "integer":
                assert np.array_equal(c_na.astype(np.float64), cref)
            else:
                assert oracle.normalised_error(c_na, cref, den) <= TOL


def test_noalloc_rejects_splits_beyond_the_array(torch_gpu):
    """An explicit split count whose partial products exceed the array is
    refused before anything is enqueued: C keeps its sentinel."""
    torch = torch_gpu
    M, N, K = 2048, 2048, 512
    assert 5 * M * N * 4 > SCRATCH_BYTES
    a, b = workloads.make_operands(M, N, K, "uniform", 3200)
    da, db, dc = _device(torch, a, b, N)
    st = dft.gemm_f32_splitk_noalloc(M, N, K, da.data_ptr(), K, db.data_ptr(), N, dc.data_ptr(), N, 5,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == dft.GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert np.all(dc.cpu().numpy().view(np.uint32) == SENTINEL_BITS)
