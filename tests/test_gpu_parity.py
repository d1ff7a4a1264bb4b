"""Parity of the HIP kernels with the fp64 CPU oracle, through the C ABI.

Bar (from the method's own pass criterion): max |C - Cref| / (|A||B|)_ij
<= 1e-5 per element, full comparison for the small and deep-K shapes and
sampled rows and columns (64 of each, always including the first and last)
for the 4096^3 and 8192^3 squares.  Integer-valued operands (entries in
{-4..4}) make every partial sum exact in fp32, so there the GPU result must
equal the oracle bit for bit in any summation order.
"""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5
SENTINEL_BITS = np.uint32(0x7FC0DEAD)  # a quiet NaN with a recognisable payload
SENTINEL = SENTINEL_BITS.view(np.float32)

ALL_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA, dft.VARIANT_VALU, dft.VARIANT_MFMA_STAGES1,
                dft.VARIANT_MFMA_NOPAD, dft.VARIANT_MFMA_SCALAR, dft.VARIANT_MFMA16, dft.VARIANT_MFMA_128,
                dft.VARIANT_MFMA_128_BK32, dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA_128_DIRECT,
                dft.VARIANT_MFMA_128_BK32_DIRECT, dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_256x256_DIRECT,
                dft.VARIANT_MFMA_256x256_W4_DIRECT, dft.VARIANT_MFMA_256x256_PIPE, dft.VARIANT_MFMA_256x256_BK32_PIPE,
    dft.VARIANT_MFMA16_256x256_DIRECT, dft.VARIANT_MFMA16_256x256_W4_BK32_PIPE, dft.VARIANT_MFMA_64_BK32_DIRECT,
    dft.VARIANT_MFMA_64_KS4, dft.VARIANT_MFMA_32x64_KS4, dft.VARIANT_MFMA_32x32_KS8,
    dft.VARIANT_MFMA_64_BK32_PIPE, dft.VARIANT_MFMA_64_KS2]
VARIANT_IDS = [dft.VARIANT_NAMES[v] for v in ALL_VARIANTS]


@pytest.fixture(scope="module")
def torch_gpu(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected a gfx950 device, found {name}"
    return torch


def test_one_hip_runtime_in_the_process(torch_gpu):
    """The library must share torch's HIP runtime (one libamdhip64 mapped)."""
    torch_gpu.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read().splitlines()
    runtimes = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(runtimes) == 1, runtimes


def run_gemm(torch, a: np.ndarray, b: np.ndarray, variant: int, lda=None, ldb=None, ldc=None,
             offset: int = 0, stream=None, c_rows_extra: int = 1):
    """Copy a, b into (possibly padded) device buffers, run the GEMM, return
    (C, full C buffer as a rows x ldc array).  The C buffer is pre-filled with
    a NaN sentinel; `offset` shifts every operand by that many floats."""
    M, K = a.shape
    N = b.shape[1]
    lda = lda or max(K, 1)
    ldb = ldb or max(N, 1)
    ldc = ldc or max(N, 1)
    abuf = np.concatenate([np.full(offset, SENTINEL, np.float32), workloads.embed(a, lda, SENTINEL)])
    bbuf = np.concatenate([np.full(offset, SENTINEL, np.float32), workloads.embed(b, ldb, SENTINEL)])
    cbuf = np.full(offset + (M + c_rows_extra) * ldc, SENTINEL, np.float32)
    da, db, dc = (torch.from_numpy(x).cuda() for x in (abuf, bbuf, cbuf))
    handle = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    st = dft.gemm_f32_ex(M, N, K, da.data_ptr() + 4 * offset, lda, db.data_ptr() + 4 * offset, ldb,
                         dc.data_ptr() + 4 * offset, ldc, handle, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    full = dc.cpu().numpy()[offset:].reshape(M + c_rows_extra, ldc)
    return full[:M, :N].copy(), full


def check_sentinels(full: np.ndarray, M: int, N: int):
    bits = full.view(np.uint32)
    outside = np.ones(full.shape, bool)
    outside[:M, :N] = False
    assert np.all(bits[outside] == SENTINEL_BITS), "a write landed outside the M x N region"


_oracle_cache: dict = {}


def reference_for(cfg: workloads.GemmConfig, integer: bool):
    key = (cfg.name, integer)
    if key not in _oracle_cache:
        a, b = workloads.config_operands(cfg, integer=integer)
        if cfg.sampled:
            rows, cols = workloads.sample_rows_cols(cfg)
            ref = (oracle.reference(a, b, rows=rows), oracle.reference(a, b, cols=cols), rows, cols)
        else:
            ref = (oracle.reference(a, b),)
        _oracle_cache[key] = (a, b, ref)
    return _oracle_cache[key]


def compare(cfg, c: np.ndarray, ref, exact: bool) -> float:
    if cfg.sampled:
        (cr, dr), (cc, dc), rows, cols = ref
        pairs = [(c[rows, :], cr, dr), (c[:, cols], cc, dc)]
    else:
        (cf, df), = ref
        pairs = [(c, cf, df)]
    if exact:
        for got, want, _ in pairs:
            assert np.array_equal(got.astype(np.float64), want), "integer-valued product differs"
        return 0.0
    return max(oracle.normalised_error(got, want, den) for got, want, den in pairs)


CONFIG_ORDER = ["small128", "ragged", "deepk", "shard8_4096", "square4096", "square8192"]


@pytest.mark.parametrize("cfg_name", CONFIG_ORDER)
@pytest.mark.parametrize("variant", ALL_VARIANTS, ids=VARIANT_IDS)
def test_config_parity(cfg_name, variant, torch_gpu):
    cfg = workloads.CONFIG_BY_NAME[cfg_name]
    a, b, ref = reference_for(cfg, integer=False)
    c, full = run_gemm(torch_gpu, a, b, variant)
    check_sentinels(full, cfg.M, cfg.N)
    err = compare(cfg, c, ref, exact=False)
    print(f"{cfg_name} {dft.VARIANT_NAMES[variant]}: normalised error {err:.3e}")
    assert err <= TOL


FULL_CHECK_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA, dft.VARIANT_VALU]


@pytest.mark.parametrize("variant", FULL_CHECK_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in FULL_CHECK_VARIANTS])
def test_square4096_every_element(variant, torch_gpu):
    """The headline shape checked on all 16.8 M outputs, not a sample (the
    oracle's 6.9e10 multiply-adds take a few seconds on the host's cores)."""
    cfg = workloads.CONFIG_BY_NAME["square4096"]
    key = ("square4096", "full")
    if key not in _oracle_cache:
        a, b = workloads.config_operands(cfg, integer=False)
        _oracle_cache[key] = (a, b, oracle.reference(a, b))
    a, b, (cref, den) = _oracle_cache[key]
    c, _ = run_gemm(torch_gpu, a, b, variant)
    err = oracle.normalised_error(c, cref, den)
    print(f"square4096 {dft.VARIANT_NAMES[variant]} all elements: normalised error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("cfg_name", CONFIG_ORDER)
@pytest.mark.parametrize("variant", ALL_VARIANTS, ids=VARIANT_IDS)
def test_config_integer_exact(cfg_name, variant, torch_gpu):
    cfg = workloads.CONFIG_BY_NAME[cfg_name]
    a, b, ref = reference_for(cfg, integer=True)
    c, _ = run_gemm(torch_gpu, a, b, variant)
    compare(cfg, c, ref, exact=True)


EDGE_SHAPES = [
    (1, 1, 1), (1, 1, 17), (2, 3, 5), (3, 2, 4), (31, 33, 15), (127, 129, 15), (128, 128, 16),
    (129, 127, 17), (255, 1, 300), (1, 257, 33), (64, 64, 1), (300, 200, 48), (257, 131, 129),
    (16, 520, 64), (520, 16, 64),
]


EDGE_VARIANTS = [dft.VARIANT_MFMA, dft.VARIANT_VALU, dft.VARIANT_MFMA_STAGES1, dft.VARIANT_MFMA16,
                 dft.VARIANT_MFMA_128, dft.VARIANT_MFMA_128_BK32, dft.VARIANT_MFMA_DIRECT,
                 dft.VARIANT_MFMA_128_DIRECT, dft.VARIANT_MFMA_128_BK32_DIRECT, dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_64_BK32_DIRECT,
                 dft.VARIANT_MFMA_256x256_DIRECT] + [dft.VARIANT_MFMA_64_KS4, dft.VARIANT_MFMA_32x64_KS4, dft.VARIANT_MFMA_32x32_KS8,
                                                     dft.VARIANT_MFMA_64_KS2]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in EDGE_SHAPES])
@pytest.mark.parametrize("variant", EDGE_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in EDGE_VARIANTS])
def test_edge_shapes(shape, variant, torch_gpu):
    M, N, K = shape
    a, b = workloads.make_operands(M, N, K, "uniform", M * 7 + N * 13 + K)
    cref, den = oracle.reference(a, b)
    for offset in (0, 1):  # offset 1 float: unaligned operands take the 4-byte load path
        c, full = run_gemm(torch_gpu, a, b, variant, offset=offset)
        check_sentinels(full, M, N)
        assert oracle.normalised_error(c, cref, den) <= TOL, (shape, offset)
    ai, bi = workloads.make_operands(M, N, K, "integer", M + N + K)
    ci, _ = run_gemm(torch_gpu, ai, bi, variant)
    assert np.array_equal(ci.astype(np.float64), oracle.reference(ai, bi)[0])


@pytest.mark.parametrize("variant", [dft.VARIANT_MFMA, dft.VARIANT_VALU, dft.VARIANT_MFMA16, dft.VARIANT_MFMA_128,
                                     dft.VARIANT_MFMA_DIRECT],
                         ids=["mfma", "valu", "mfma16", "mfma_128", "mfma_direct"])
@pytest.mark.parametrize("pitch", [(3, 5, 2), (2, 4, 4), (1, 0, 9), (0, 8, 0)], ids=str)
def test_pitched_operands(pitch, variant, torch_gpu):
    """Leading dimensions beyond the width: NaN in every gap must never be
    read (the result stays finite and exact) and no gap of C is written."""
    M, N, K = 150, 140, 70
    a, b = workloads.make_operands(M, N, K, "integer", 77)
    cref, _ = oracle.reference(a, b)
    pa, pb, pc = pitch
    c, full = run_gemm(torch_gpu, a, b, variant, lda=K + pa, ldb=N + pb, ldc=N + pc, c_rows_extra=3)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref)


DIRECT_VARIANTS = [dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA_128_DIRECT, dft.VARIANT_MFMA_128_BK32_DIRECT,
                   dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_256x256_DIRECT, dft.VARIANT_MFMA_256x256_W4_DIRECT,
                   dft.VARIANT_MFMA_256x256_PIPE, dft.VARIANT_MFMA_256x256_BK32_PIPE,
    dft.VARIANT_MFMA16_256x256_DIRECT, dft.VARIANT_MFMA16_256x256_W4_BK32_PIPE, dft.VARIANT_MFMA_64_BK32_DIRECT,
    dft.VARIANT_MFMA_64_BK32_PIPE]


@pytest.mark.parametrize("variant", DIRECT_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in DIRECT_VARIANTS])
@pytest.mark.parametrize("K", [1, 15, 16, 17, 31, 32, 33, 100, 256])
def test_direct_copy_paths(K, variant, torch_gpu):
    """Direct-copy variants on a grid with interior and edge tiles (600 x 300
    is 3 x 3 tiles of 256 x 128, 5 x 3 of 128 x 128): workgroups copy whole K
    tiles global->LDS directly (edge tiles moved back to end at M or N) and
    load a ragged last K tile through registers with zero fill.  Leading
    dimensions are
    multiples of 4 with NaN in every gap, so a copy that strays past column K
    or into a gap shows up, as does any write outside C."""
    M, N = 600, 300
    lda, ldb, ldc = K + (4 - K % 4) % 4 + 4, N + 8, N + 1
    a, b = workloads.make_operands(M, N, K, "integer", 300 + K)
    cref, _ = oracle.reference(a, b)
    c, full = run_gemm(torch_gpu, a, b, variant, lda=lda, ldb=ldb, ldc=ldc, c_rows_extra=2)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref)
    au, bu = workloads.make_operands(M, N, K, "uniform", 400 + K)
    cu, _ = run_gemm(torch_gpu, au, bu, variant, lda=lda, ldb=ldb)
    cref_u, den_u = oracle.reference(au, bu)
    assert oracle.normalised_error(cu, cref_u, den_u) <= TOL


FOUR_BYTE_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_64_DIRECT, dft.VARIANT_MFMA_64_BK32_DIRECT, dft.VARIANT_MFMA_DIRECT, dft.VARIANT_MFMA_128_DIRECT,
                      dft.VARIANT_MFMA_128_BK32_DIRECT, dft.VARIANT_MFMA_256x256_BK32_PIPE]


@pytest.mark.parametrize("variant", FOUR_BYTE_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in FOUR_BYTE_VARIANTS])
@pytest.mark.parametrize("K,pad,offset", [(513, 0, 0), (100, 1, 1), (257, 2, 3), (16, 1, 0), (33, 3, 1)])
def test_four_byte_direct_copies(K, pad, offset, variant, torch_gpu):
    """Operands whose rows are not 16-byte aligned (odd leading dimensions,
    bases shifted by whole floats): the direct-copy kernels copy them into
    LDS 4 bytes per lane.  600 x 300 has interior and edge tiles for every
    tile size up to 256 x 256; NaN fills every ld gap, so a copy that strays
    past column K or into a gap shows up, as does any write outside C."""
    M, N = 600, 300
    lda, ldb, ldc = K + pad, N + 1 + pad, N + 3
    a, b = workloads.make_operands(M, N, K, "integer", 500 + K)
    cref, _ = oracle.reference(a, b)
    c, full = run_gemm(torch_gpu, a, b, variant, lda=lda, ldb=ldb, ldc=ldc, offset=offset, c_rows_extra=2)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref)


KSPLIT_VARIANTS = [dft.VARIANT_MFMA_64_KS4, dft.VARIANT_MFMA_32x64_KS4, dft.VARIANT_MFMA_32x32_KS8,
                   dft.VARIANT_MFMA_64_KS2]
PER_OPERAND_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_256x256_BK32_PIPE, dft.VARIANT_MFMA_DIRECT,
                        dft.VARIANT_MFMA_128_DIRECT, dft.VARIANT_MFMA_128_BK32_DIRECT,
                        dft.VARIANT_MFMA_64_BK32_DIRECT] + KSPLIT_VARIANTS


@pytest.mark.parametrize("variant", KSPLIT_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in KSPLIT_VARIANTS])
@pytest.mark.parametrize("K", [1, 31, 32, 33, 64, 95, 96, 160, 255, 256, 257, 1000])
def test_k_split_in_the_workgroup(K, variant, torch_gpu):
    """Wave groups splitting K inside the workgroup: K tiles are dealt to the
    groups in turn, so these K cover fewer tiles than groups, a count that
    is not a multiple of the groups, and a ragged last tile falling to any
    group; the partial sums are added in LDS.  130 x 100 spans interior and
    moved edge tiles of every tile size; bit for bit on integer operands,
    NaN in every ld gap and around C."""
    M, N = 130, 100
    lda, ldb, ldc = K + (4 - K % 4) % 4 + 4, N + 4, N + 3
    a, b = workloads.make_operands(M, N, K, "integer", 1500 + K)
    cref, _ = oracle.reference(a, b)
    c, full = run_gemm(torch_gpu, a, b, variant, lda=lda, ldb=ldb, ldc=ldc, c_rows_extra=2)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref)
    au, bu = workloads.make_operands(M, N, K, "uniform", 1600 + K)
    for offset in (0, 1):  # 1: 4-byte copies of both operands
        cu, full = run_gemm(torch_gpu, au, bu, variant, offset=offset)
        check_sentinels(full, M, N)
        cref_u, den_u = oracle.reference(au, bu)
        assert oracle.normalised_error(cu, cref_u, den_u) <= TOL, offset


@pytest.mark.parametrize("variant", PER_OPERAND_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in PER_OPERAND_VARIANTS])
@pytest.mark.parametrize("which", ["a", "b"])
@pytest.mark.parametrize("K", [16, 33, 100, 257])
def test_one_operand_unaligned(K, which, variant, torch_gpu):
    """Only A's rows (or only B's) are not 16-byte aligned: the variants
    AUTO chooses from then copy that operand 4 bytes per lane and the other
    16 bytes per lane.  600 x 520 spans interior and moved edge tiles of
    every tile size; NaN fills every ld gap, so a copy that strays past
    column K or N or into a gap shows up, as does any write outside C."""
    M, N = 600, 520
    lda = K + (4 - K % 4) % 4 + (1 if which == "a" else 4)
    ldb = N + (1 if which == "b" else 4)
    assert (lda % 4 != 0) == (which == "a") and (ldb % 4 != 0) == (which == "b")
    a, b = workloads.make_operands(M, N, K, "integer", 1300 + K)
    cref, _ = oracle.reference(a, b)
    c, full = run_gemm(torch_gpu, a, b, variant, lda=lda, ldb=ldb, ldc=N + 3, c_rows_extra=2)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref)
    au, bu = workloads.make_operands(M, N, K, "uniform", 1400 + K)
    cu, _ = run_gemm(torch_gpu, au, bu, variant, lda=lda, ldb=ldb)
    cref_u, den_u = oracle.reference(au, bu)
    assert oracle.normalised_error(cu, cref_u, den_u) <= TOL


MOVED_SHAPES = [(65, 70, 64), (129, 250, 96), (257, 300, 64), (300, 257, 33), (511, 767, 100), (520, 260, 32),
                (256, 257, 40), (257, 256, 40)]
MOVED_VARIANTS = [dft.VARIANT_AUTO] + DIRECT_VARIANTS


@pytest.mark.parametrize("variant", MOVED_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in MOVED_VARIANTS])
@pytest.mark.parametrize("shape", MOVED_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in MOVED_SHAPES])
def test_moved_edge_tiles(shape, variant, torch_gpu):
    """Shapes a little past one or more whole tiles in M and/or N: a
    direct-copy workgroup whose tile overhangs M (N) computes the tile that
    ends at M (N) instead, overlapping its neighbour, and stores only the rows
    and columns it owns.  Checked bit for bit on integer operands (a tile
    moved by the wrong amount gives wrong sums) and to the tolerance on
    uniform ones, with aligned and 4-byte-offset operands, a padded C and
    NaN around every operand, so a stray copy or write shows up."""
    M, N, K = shape
    a, b = workloads.make_operands(M, N, K, "integer", 900 + M + N + K)
    cref, _ = oracle.reference(a, b)
    for offset in (0, 1):
        c, full = run_gemm(torch_gpu, a, b, variant, lda=K + 4, ldb=N + 4, ldc=N + 5, offset=offset,
                           c_rows_extra=2)
        check_sentinels(full, M, N)
        assert np.array_equal(c.astype(np.float64), cref), (shape, offset)
    au, bu = workloads.make_operands(M, N, K, "uniform", 950 + M + N + K)
    cu, _ = run_gemm(torch_gpu, au, bu, variant)
    cref_u, den_u = oracle.reference(au, bu)
    assert oracle.normalised_error(cu, cref_u, den_u) <= TOL


PITCH_SHAPES = [(129, 250, 96), (257, 301, 40), (520, 263, 33), (300, 1003, 64)]


@pytest.mark.parametrize("variant", MOVED_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in MOVED_VARIANTS])
@pytest.mark.parametrize("shape", PITCH_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in PITCH_SHAPES])
def test_moved_edge_tiles_with_aligned_pitch(shape, variant, torch_gpu):
    """B's rows start 16-byte aligned (ldb a multiple of 4) but N is not a
    multiple of 4: an edge tile moved back to end at N starts its B columns
    at N - BN, off a 16-byte boundary, so B must be copied 4 bytes per lane.
    Bit for bit on integer operands, NaN in every gap and around C."""
    M, N, K = shape
    assert N % 4
    lda, ldb = K + (-K) % 4 + 4, N + (-N) % 4 + 4
    assert lda % 4 == 0 and ldb % 4 == 0
    a, b = workloads.make_operands(M, N, K, "integer", 1700 + M + N + K)
    cref, _ = oracle.reference(a, b)
    c, full = run_gemm(torch_gpu, a, b, variant, lda=lda, ldb=ldb, ldc=N + 3, c_rows_extra=2)
    check_sentinels(full, M, N)
    assert np.array_equal(c.astype(np.float64), cref), shape


@pytest.mark.parametrize("variant", ALL_VARIANTS, ids=VARIANT_IDS)
def test_k_zero_writes_zeros(variant, torch_gpu):
    a = np.zeros((37, 0), np.float32)
    b = np.zeros((0, 45), np.float32)
    c, full = run_gemm(torch_gpu, a, b, variant, ldc=50)
    check_sentinels(full, 37, 45)
    assert np.array_equal(c, np.zeros((37, 45), np.float32))


def test_empty_m_or_n_touches_nothing(torch_gpu):
    torch = torch_gpu
    cbuf = torch.from_numpy(np.full(64, SENTINEL, np.float32)).cuda()
    a = torch.ones(16, device="cuda")
    b = torch.ones(16, device="cuda")
    for (M, N, K) in [(0, 4, 4), (4, 0, 4), (0, 0, 0)]:
        st = dft.gemm_f32(M, N, K, a.data_ptr(), max(K, 1), b.data_ptr(), max(N, 1), cbuf.data_ptr(),
                          max(N, 1), None)
        assert st == dft.GEMM_OK
    torch.cuda.synchronize()
    assert np.all(cbuf.cpu().numpy().view(np.uint32) == SENTINEL_BITS)


def test_tall_and_wide(torch_gpu):
    for (M, N, K) in [(70000, 3, 7), (2, 100003, 9), (1, 1, 70001)]:
        a, b = workloads.make_operands(M, N, K, "integer", 5)
        c, _ = run_gemm(torch_gpu, a, b, dft.VARIANT_AUTO)
        assert np.array_equal(c.astype(np.float64), oracle.reference(a, b)[0]), (M, N, K)


def test_deterministic_and_stream_ordered(torch_gpu):
    torch = torch_gpu
    cfg = workloads.CONFIG_BY_NAME["ragged"]
    a, b = workloads.config_operands(cfg)
    c0, _ = run_gemm(torch, a, b, dft.VARIANT_MFMA)
    s = torch.cuda.Stream()
    c1, _ = run_gemm(torch, a, b, dft.VARIANT_MFMA, stream=s)
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))


def test_matmul_wrapper(torch_gpu):
    torch = torch_gpu
    a, b = workloads.make_operands(200, 300, 100, "uniform", 9)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    c = dft.matmul(ta, tb).cpu().numpy()
    cref, den = oracle.reference(a, b)
    assert oracle.normalised_error(c, cref, den) <= TOL
    # a strided view (row pitch > width) goes through as lda
    big = torch.from_numpy(workloads.embed(a, 128).reshape(200, 128)).cuda()
    c2 = dft.matmul(big[:, :100], tb).cpu().numpy()
    assert np.array_equal(c, c2)
    with pytest.raises(TypeError):
        dft.matmul(ta.double(), tb)
    with pytest.raises(ValueError):
        dft.matmul(ta, tb[:50])


def test_rejects_overlap_on_device(torch_gpu):
    torch = torch_gpu
    buf = torch.zeros(64 * 64, device="cuda")
    p = buf.data_ptr()
    st = dft.gemm_f32(8, 8, 8, p, 8, p + 4 * 64, 8, p + 4 * 32, 8, None)
    assert st == dft.GEMM_ERR_ALIAS


# ---- split-K ----
def run_splitk(torch, a, b, splits, ldc=None, ws_elems=None, variant=dft.VARIANT_AUTO):
    M, K = a.shape
    N = b.shape[1]
    ldc = ldc or max(N, 1)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    dc = torch.from_numpy(np.full((M + 1) * ldc, SENTINEL, np.float32)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = dft.gemm_f32_splitk_workspace_bytes(M, N, K, splits, cus)
    ws = torch.full((max(need // 4, 1) if ws_elems is None else ws_elems,), float("nan"), device="cuda")
    st = dft.gemm_f32_splitk_ex(M, N, K, da.data_ptr(), max(K, 1), db.data_ptr(), max(N, 1), dc.data_ptr(), ldc,
                                ws.data_ptr(), ws.numel() * 4, splits, torch.cuda.current_stream().cuda_stream,
                                variant)
    torch.cuda.synchronize()
    if st != dft.GEMM_OK:
        return st, None, None
    full = dc.cpu().numpy().reshape(M + 1, ldc)
    return st, full[:M, :N].copy(), full


SPLITK_VARIANTS = [dft.VARIANT_AUTO, dft.VARIANT_MFMA_128, dft.VARIANT_MFMA_128_BK32_DIRECT, dft.VARIANT_MFMA_DIRECT,
                   dft.VARIANT_VALU, dft.VARIANT_MFMA_64_BK32_DIRECT, dft.VARIANT_MFMA_32x64_KS4]


@pytest.mark.parametrize("variant", SPLITK_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in SPLITK_VARIANTS])
@pytest.mark.parametrize("splits", [0, 2, 7, 32, 64])
def test_splitk_deepk_parity(splits, variant, torch_gpu):
    cfg = workloads.CONFIG_BY_NAME["deepk"]
    a, b, ref = reference_for(cfg, integer=False)
    st, c, full = run_splitk(torch_gpu, a, b, splits, variant=variant)
    assert st == dft.GEMM_OK
    check_sentinels(full, cfg.M, cfg.N)
    err = compare(cfg, c, ref, exact=False)
    print(f"deepk split-K {splits} {dft.VARIANT_NAMES[variant]}: normalised error {err:.3e}")
    assert err <= TOL
    ai, bi, refi = reference_for(cfg, integer=True)
    st, ci, _ = run_splitk(torch_gpu, ai, bi, splits, variant=variant)
    compare(cfg, ci, refi, exact=True)


@pytest.mark.parametrize("variant", SPLITK_VARIANTS, ids=[dft.VARIANT_NAMES[v] for v in SPLITK_VARIANTS])
@pytest.mark.parametrize("shape", [(1000, 999, 513), (129, 127, 17), (300, 200, 48), (64, 64, 1), (5, 7, 4097),
                                   (520, 260, 1000)], ids=str)
@pytest.mark.parametrize("splits", [1, 3, 8, 64])
def test_splitk_ragged_and_empty_slices(shape, splits, variant, torch_gpu):
    """Slices past the end of K (e.g. K = 17 in 8 slices of 16) add zero."""
    M, N, K = shape
    a, b = workloads.make_operands(M, N, K, "uniform", M + 3 * N + K)
    cref, den = oracle.reference(a, b)
    st, c, full = run_splitk(torch_gpu, a, b, splits, ldc=N + 3, variant=variant)
    assert st == dft.GEMM_OK
    check_sentinels(full, M, N)
    assert oracle.normalised_error(c, cref, den) <= TOL


def test_splitk_is_deterministic(torch_gpu):
    cfg = workloads.CONFIG_BY_NAME["deepk"]
    a, b, _ = reference_for(cfg, integer=False)
    _, c0, _ = run_splitk(torch_gpu, a, b, 16)
    _, c1, _ = run_splitk(torch_gpu, a, b, 16)
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))


def test_splitk_rejects_small_workspace(torch_gpu):
    a, b = workloads.make_operands(256, 256, 1024, "uniform", 1)
    st, _, _ = run_splitk(torch_gpu, a, b, 4, ws_elems=4 * 256 * 256 - 1)
    assert st == dft.GEMM_ERR_WORKSPACE


def test_matmul_splitk_wrapper(torch_gpu):
    torch = torch_gpu
    a, b = workloads.make_operands(300, 130, 5000, "uniform", 2)
    c = dft.matmul_splitk(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy()
    cref, den = oracle.reference(a, b)
    assert oracle.normalised_error(c, cref, den) <= TOL
