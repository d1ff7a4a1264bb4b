"""Seeded random shapes, concurrent streams and HIP-graph replay, against the
fp64 oracle.  GPU only.

* Random shapes: 60 seeded (M, N, K, padding, misalignment) cases over the
  main variants, each checked to the 1e-5 bound.
* Streams: the library keeps no per-call state, so GEMMs enqueued on two
  streams at once must both be right.
* Graphs: the entry points enqueue only kernels (no memset or copy nodes),
  so a call captured in a HIP graph must replay to the same result; every
  replay is checked against the eager result, with other work in between.
"""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def torch_gpu(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    return torch


def random_cases(count: int, seed: int):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        M, N, K = (int(x) for x in rng.integers(1, 700, 3))
        pad = tuple(int(x) for x in rng.integers(0, 9, 3))
        shift = int(rng.integers(0, 2))  # 1: operands start 4 bytes off 16-byte alignment
        yield M, N, K, pad, shift


RANDOM_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_256x256_DIRECT, dft.VARIANT_MFMA_256x256_PIPE,
                   dft.VARIANT_MFMA_256x256_BK32_PIPE, dft.VARIANT_MFMA_DIRECT,
                   dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_64_BK32_DIRECT, dft.VARIANT_MFMA, dft.VARIANT_VALU,
                   dft.VARIANT_MFMA_64_KS4, dft.VARIANT_MFMA_32x64_KS4, dft.VARIANT_MFMA_32x32_KS8]


_refs: dict = {}


@pytest.mark.parametrize("variant", RANDOM_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in RANDOM_VARIANTS])
def test_random_shapes(variant, torch_gpu):
    torch = torch_gpu
    for i, (M, N, K, (pa, pb, pc), shift) in enumerate(random_cases(60, 2024)):
        a, b = workloads.make_operands(M, N, K, "uniform", 5000 + i)
        if i not in _refs:
            _refs[i] = oracle.reference(a, b)
        cref, den = _refs[i]
        lda, ldb, ldc = K + pa, N + pb, N + pc
        abuf = np.concatenate([np.zeros(shift, np.float32), workloads.embed(a, lda)])
        bbuf = np.concatenate([np.zeros(shift, np.float32), workloads.embed(b, ldb)])
        da, db = torch.from_numpy(abuf).cuda(), torch.from_numpy(bbuf).cuda()
        dc = torch.full((M * ldc,), float("nan"), device="cuda")
        st = dft.gemm_f32_ex(M, N, K, da.data_ptr() + 4 * shift, lda, db.data_ptr() + 4 * shift, ldb, dc.data_ptr(),
                             ldc, torch.cuda.current_stream().cuda_stream, variant)
        assert st == dft.GEMM_OK, (M, N, K, st)
        c = dc.cpu().numpy().reshape(M, ldc)[:, :N]
        err = oracle.normalised_error(c, cref, den)
        assert err <= TOL, (M, N, K, pa, pb, pc, shift, err)


def test_two_streams_at_once(torch_gpu):
    torch = torch_gpu
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    a1, b1 = workloads.make_operands(1024, 768, 512, "integer", 71)
    a2, b2 = workloads.make_operands(700, 900, 1300, "integer", 72)
    d = [torch.from_numpy(x).cuda() for x in (a1, b1, a2, b2)]
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            c1 = dft.matmul(d[0], d[1], stream=s1)
        with torch.cuda.stream(s2):
            c2 = dft.matmul(d[2], d[3], stream=s2)
        outs.append((c1, c2))
    torch.cuda.synchronize()
    r1, r2 = oracle.reference(a1, b1)[0], oracle.reference(a2, b2)[0]
    for c1, c2 in outs:
        assert np.array_equal(c1.cpu().numpy().astype(np.float64), r1)
        assert np.array_equal(c2.cpu().numpy().astype(np.float64), r2)


def test_graph_replay_default_path(torch_gpu):
    torch = torch_gpu
    M, N, K = 1000, 520, 700
    a, b = workloads.make_operands(M, N, K, "uniform", 81)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    c = torch.empty((M, N), device="cuda")
    eager = dft.matmul(da, db).cpu().numpy()
    cref, den = oracle.reference(a, b)
    assert oracle.normalised_error(eager, cref, den) <= TOL
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dft.matmul(da, db, out=c, stream=s)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dft.matmul(da, db, out=c, stream=s)
    for i in range(3):
        c.fill_(float("nan"))
        junk = dft.matmul(da, db)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), eager), f"replay {i} differs from the eager result"
        del junk


def test_graph_replay_splitk(torch_gpu):
    """Split-K is two kernels (slices, then the ordered reduction) with a
    caller workspace; both must be captured and replay exactly."""
    torch = torch_gpu
    M, N, K = 512, 256, 8192
    a, b = workloads.make_operands(M, N, K, "uniform", 91)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = dft.gemm_f32_splitk_workspace_bytes(M, N, K, 8, cus)
    ws = torch.empty(need // 4, device="cuda")
    c = torch.empty((M, N), device="cuda")
    eager = dft.matmul_splitk(da, db, splits=8, workspace=ws).cpu().numpy()
    cref, den = oracle.reference(a, b)
    assert oracle.normalised_error(eager, cref, den) <= TOL
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dft.matmul_splitk(da, db, out=c, splits=8, workspace=ws, stream=s)
    for i in range(3):
        c.fill_(float("nan"))
        ws.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), eager), f"replay {i} differs from the eager result"
