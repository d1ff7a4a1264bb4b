"""Every kernel reads only LDS words that the same workgroup wrote.

The library's debug build (libdense_fp32_tiled_poison.so, compiled with
DFT_LDS_POISON=1) fills each workgroup's whole LDS allocation with a quiet
NaN (0x7FC07FC0: NaN as fp32, and in both halves as bf16 or fp16) before
its first copy.  A multiply that reads a word no copy wrote (a K tail past
the last copied column, a moved edge tile's rows, a 4-byte or 2-byte copy
that skips a word, a pad column, the other group's half of a K-split
reduction) then spreads NaN into C, where a zero-initialised or stale LDS
would hide it.  Run through the poison build's own C ABI handle, every
variant on shapes with ragged M, N and K, moved edge tiles, unaligned
rows and K-split tails: bit for bit against the fp64 oracle on
integer-valued operands, NaN in every ld gap and around C.
"""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads
from dense_fp32_tiled_amd import build

pytestmark = pytest.mark.gpu

SENTINEL_BITS = np.uint32(0x7FC0DEAD)
SENTINEL = SENTINEL_BITS.view(np.float32)
NAN16 = {"bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}
TYPES = {"bf16": dft.INPUT_BF16, "f16": dft.INPUT_F16}

# (M, N, K, extra lda, extra ldb, base offset in elements)
F32_CASES = [
    (1, 1, 1, 0, 0, 0),
    (65, 70, 33, 3, 2, 0),      # ragged K tail, moved tiles in M and N
    (129, 250, 96, 4, 4, 0),    # aligned rows, moved edge tiles
    (300, 257, 33, 1, 1, 1),    # 4-byte copies of both operands
    (130, 100, 1000, 4, 4, 0),  # K-split groups with a ragged last tile
    (520, 263, 513, 0, 4, 0),   # odd K: A copied 4 bytes per lane
    (257, 256, 40, 4, 1, 0),    # only B unaligned
    (64, 64, 1, 4, 4, 0),       # one K column
]
MIXED_CASES = [
    (1, 1, 1, 0, 0, 0),
    (31, 33, 15, 0, 0, 0),      # odd K and N: 2-byte loads
    (257, 255, 33, 0, 0, 1),
    (300, 260, 130, 2, 4, 0),   # 4-byte copies
    (300, 520, 100, 4, 8, 0),   # aligned rows, moved edge tiles
    (130, 100, 1000, 8, 4, 0),  # K-split groups
    (300, 250, 100, 4, 6, 0),   # ldb aligned, N not: narrow copies of moved B
    (300, 260, 33, 1, 1, 0),    # rows 2-byte aligned: raw copies realigned in LDS
    (520, 300, 64, 3, 1, 1),
    (256, 256, 1, 1, 1, 0),
]

_refs: dict = {}


@pytest.fixture(scope="module")
def poison(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    return torch, dft.library(build.POISON_LIB)


def case_id(case) -> str:
    M, N, K, pa, pb, off = case
    return f"{M}x{N}x{K}_lda+{pa}_ldb+{pb}_off{off}"


def integer_case(M, N, K, kind=None):
    key = (M, N, K, kind)
    if key not in _refs:
        a, b = workloads.make_operands(M, N, K, "integer", 7000 + M + 3 * N + 7 * K)
        if kind is None:
            _refs[key] = (a, b, oracle.reference(a, b)[0])
        else:
            (ab, af), (bb, bf) = workloads.to_16bit(a, kind), workloads.to_16bit(b, kind)
            _refs[key] = (ab, bb, oracle.reference(af, bf)[0])
    return _refs[key]


def check_c(dc, M, N, ldc, cref):
    full = dc.cpu().numpy().reshape(M + 2, ldc)
    outside = np.ones(full.shape, bool)
    outside[:M, :N] = False
    assert np.all(full.view(np.uint32)[outside] == SENTINEL_BITS), "a write landed outside the M x N region"
    c = full[:M, :N].astype(np.float64)
    assert not np.isnan(c).any(), f"{int(np.isnan(c).sum())} NaN outputs: a read of LDS that no copy wrote"
    assert np.array_equal(c, cref)


@pytest.mark.parametrize("case", F32_CASES, ids=[case_id(c) for c in F32_CASES])
@pytest.mark.parametrize("variant", range(dft.VARIANT_COUNT), ids=[dft.VARIANT_NAMES[v] for v in
                                                                    range(dft.VARIANT_COUNT)])
def test_f32_kernels_read_only_written_lds(case, variant, poison):
    torch, lib = poison
    M, N, K, pa, pb, off = case
    a, b, cref = integer_case(M, N, K)
    lda, ldb, ldc = K + pa, N + pb, N + 3
    abuf = np.concatenate([np.full(off, SENTINEL, np.float32), workloads.embed(a, lda, SENTINEL)])
    bbuf = np.concatenate([np.full(off, SENTINEL, np.float32), workloads.embed(b, ldb, SENTINEL)])
    da, db = torch.from_numpy(abuf).cuda(), torch.from_numpy(bbuf).cuda()
    dc = torch.from_numpy(np.full((M + 2) * ldc, SENTINEL, np.float32)).cuda()
    st = lib.gemm_f32_ex(M, N, K, da.data_ptr() + 4 * off, lda, db.data_ptr() + 4 * off, ldb, dc.data_ptr(), ldc,
                         torch.cuda.current_stream().cuda_stream, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    check_c(dc, M, N, ldc, cref)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("case", F32_CASES[1:6], ids=[case_id(c) for c in F32_CASES[1:6]])
def test_splitk_reads_only_written_lds(case, splits, poison):
    """Split-K: each slice's kernel runs on a K range that starts mid-matrix
    and may end in a ragged tile."""
    torch, lib = poison
    M, N, K, pa, pb, off = case
    a, b, cref = integer_case(M, N, K)
    lda, ldb, ldc = K + pa, N + pb, N + 3
    da = torch.from_numpy(workloads.embed(a, lda, SENTINEL)).cuda()
    db = torch.from_numpy(workloads.embed(b, ldb, SENTINEL)).cuda()
    dc = torch.from_numpy(np.full((M + 2) * ldc, SENTINEL, np.float32)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = dft.gemm_f32_splitk_workspace_bytes(M, N, K, splits, cus)
    ws = torch.full((max(need // 4, 1),), float("nan"), device="cuda")
    st = lib.gemm_f32_splitk_ex(M, N, K, da.data_ptr(), lda, db.data_ptr(), ldb, dc.data_ptr(), ldc, ws.data_ptr(),
                                ws.numel() * 4, splits, torch.cuda.current_stream().cuda_stream, dft.VARIANT_AUTO)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    check_c(dc, M, N, ldc, cref)


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("case", MIXED_CASES, ids=[case_id(c) for c in MIXED_CASES])
@pytest.mark.parametrize("variant", range(dft.MIXED_COUNT), ids=[dft.MIXED_NAMES[v] for v in
                                                                  range(dft.MIXED_COUNT)])
def test_mixed_kernels_read_only_written_lds(kind, case, variant, poison):
    torch, lib = poison
    M, N, K, pa, pb, off = case
    ab, bb, cref = integer_case(M, N, K, kind)
    lda, ldb, ldc = K + pa, N + pb, N + 3

    def buf(bits, ld):
        out = np.full((max(bits.shape[0], 1), ld), NAN16[kind], np.uint16)
        out[:bits.shape[0], :bits.shape[1]] = bits
        return np.concatenate([np.full(off, NAN16[kind], np.uint16), out.reshape(-1)]).view(np.int16)

    da, db = torch.from_numpy(buf(ab, lda)).cuda(), torch.from_numpy(buf(bb, ldb)).cuda()
    dc = torch.from_numpy(np.full((M + 2) * ldc, SENTINEL, np.float32)).cuda()
    st = lib.gemm_mixed_f32(TYPES[kind], M, N, K, da.data_ptr() + 2 * off, lda, db.data_ptr() + 2 * off, ldb,
                            dc.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    check_c(dc, M, N, ldc, cref)
