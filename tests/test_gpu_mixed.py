"""GPU parity of the 16-bit-input kernels (gemm_mixed_f32: bf16 or fp16 A and
B, fp32 accumulation and C) against the fp64 oracle.

The oracle multiplies the exact float32 widenings of the 16-bit inputs, so
the GPU result differs from it only by fp32 accumulation: the fp32 bar
applies (normalised error <= 1e-5), and integer-valued inputs must match bit
for bit.  Buffers carry NaN in every ld gap and around C."""

from __future__ import annotations

import numpy as np
import pytest

import dense_fp32_tiled_amd as dft
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-5
SENTINEL_BITS = np.uint32(0x7FC0DEAD)
NAN16 = {"bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}
TYPES = {"bf16": dft.INPUT_BF16, "f16": dft.INPUT_F16}
VARIANTS = list(range(dft.MIXED_COUNT))
VARIANT_IDS = [dft.MIXED_NAMES[v] for v in VARIANTS]


@pytest.fixture(scope="module")
def torch_gpu(gemm_lib):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    return torch


def embed16(bits: np.ndarray, ld: int, fill: np.uint16) -> np.ndarray:
    rows, cols = bits.shape
    out = np.full((max(rows, 1), ld), fill, dtype=np.uint16)
    out[:rows, :cols] = bits
    return out.reshape(-1)


def run_mixed(torch, kind, a_bits, b_bits, variant, lda=None, ldb=None, ldc=None, offset=0):
    M, K = a_bits.shape
    N = b_bits.shape[1]
    lda, ldb, ldc = lda or max(K, 1), ldb or max(N, 1), ldc or max(N, 1)
    pad = np.full(offset, NAN16[kind], np.uint16)
    abuf = np.concatenate([pad, embed16(a_bits, lda, NAN16[kind])]).view(np.int16)
    bbuf = np.concatenate([pad, embed16(b_bits, ldb, NAN16[kind])]).view(np.int16)
    cbuf = np.full((M + 1) * ldc, SENTINEL_BITS, np.uint32).view(np.float32)
    da, db, dc = (torch.from_numpy(x).cuda() for x in (abuf, bbuf, cbuf))
    st = dft.gemm_mixed_f32(TYPES[kind], M, N, K, da.data_ptr() + 2 * offset, lda, db.data_ptr() + 2 * offset, ldb,
                            dc.data_ptr(), ldc, torch.cuda.current_stream().cuda_stream, variant)
    assert st == dft.GEMM_OK, dft.gemm_f32_status_string(st)
    torch.cuda.synchronize()
    full = dc.cpu().numpy().reshape(M + 1, ldc)
    outside = np.ones(full.shape, bool)
    outside[:M, :N] = False
    assert np.all(full.view(np.uint32)[outside] == SENTINEL_BITS), "a write landed outside the M x N region"
    return full[:M, :N].copy()


def operands(kind, M, N, K, dist, seed):
    a, b = workloads.make_operands(M, N, K, dist, seed)
    (ab, af), (bb, bf) = workloads.to_16bit(a, kind), workloads.to_16bit(b, kind)
    return ab, bb, af, bf


_cache: dict = {}


def reference(kind, cfg, integer):
    key = (kind, cfg.name, integer)
    if key not in _cache:
        seed = cfg.seed + (workloads.INTEGER_SEED_OFFSET if integer else 0)
        ab, bb, af, bf = operands(kind, cfg.M, cfg.N, cfg.K, "integer" if integer else cfg.dist, seed)
        if cfg.sampled:
            rows, cols = workloads.sample_rows_cols(cfg)
            ref = (oracle.reference(af, bf, rows=rows), oracle.reference(af, bf, cols=cols), rows, cols)
        else:
            ref = (oracle.reference(af, bf),)
        _cache[key] = (ab, bb, ref)
    return _cache[key]


def compare(cfg, c, ref, exact):
    if cfg.sampled:
        (cr, dr), (cc, dcol), rows, cols = ref
        pairs = [(c[rows, :], cr, dr), (c[:, cols], cc, dcol)]
    else:
        (cf, df), = ref
        pairs = [(c, cf, df)]
    if exact:
        for got, want, _ in pairs:
            assert np.array_equal(got.astype(np.float64), want), "integer-valued product differs"
        return 0.0
    return max(oracle.normalised_error(got, want, den) for got, want, den in pairs)


CONFIGS = ["small128", "ragged", "deepk", "shard8_4096", "square4096"]


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("cfg_name", CONFIGS)
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_mixed_config_parity(kind, cfg_name, variant, torch_gpu):
    cfg = workloads.CONFIG_BY_NAME[cfg_name]
    ab, bb, ref = reference(kind, cfg, integer=False)
    c = run_mixed(torch_gpu, kind, ab, bb, variant)
    err = compare(cfg, c, ref, exact=False)
    print(f"{kind} {cfg_name} {dft.MIXED_NAMES[variant]}: normalised error {err:.3e}")
    assert err <= TOL
    abi, bbi, refi = reference(kind, cfg, integer=True)
    compare(cfg, run_mixed(torch_gpu, kind, abi, bbi, variant), refi, exact=True)


EDGE_SHAPES = [(1, 1, 1), (2, 3, 5), (31, 33, 15), (127, 129, 17), (256, 256, 32), (257, 255, 33), (300, 520, 100),
               (520, 16, 64), (16, 520, 64), (600, 300, 1000)]


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in EDGE_SHAPES])
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_mixed_edge_shapes(kind, shape, variant, torch_gpu):
    """Ragged shapes, aligned (direct copies for in-range tiles) and shifted
    by one element (2-byte loads), with padded leading dimensions."""
    M, N, K = shape
    ab, bb, af, bf = operands(kind, M, N, K, "uniform", M * 7 + N * 13 + K)
    cref, den = oracle.reference(af, bf)
    pad_a, pad_b = (8 - K % 8) % 8 + 8, (8 - N % 8) % 8 + 8
    for offset, lda, ldb in ((0, K + pad_a, N + pad_b), (1, None, None)):
        c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=lda, ldb=ldb, ldc=N + 3, offset=offset)
        assert oracle.normalised_error(c, cref, den) <= TOL, (shape, offset)
    abi, bbi, afi, bfi = operands(kind, M, N, K, "integer", M + N + K)
    ci = run_mixed(torch_gpu, kind, abi, bbi, variant)
    assert np.array_equal(ci.astype(np.float64), oracle.reference(afi, bfi)[0])


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("K,pad_a,pad_b,offset", [(130, 2, 4, 0), (64, 6, 2, 2), (200, 4, 6, 2), (1000, 2, 2, 0)])
def test_mixed_four_byte_copies(kind, K, pad_a, pad_b, offset, variant, torch_gpu):
    """Rows 4-byte but not 16-byte aligned (even leading dimensions not a
    multiple of 8, bases shifted by two elements): the variants copy two
    elements per lane.  Bit for bit on integer operands, within the bar on
    uniform ones; NaN fills every ld gap."""
    M, N = 300, 260
    lda, ldb = K + pad_a, N + pad_b
    assert lda % 2 == 0 and ldb % 2 == 0 and (lda % 8 or ldb % 8 or offset)
    ab, bb, af, bf = operands(kind, M, N, K, "integer", 1900 + K)
    c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=lda, ldb=ldb, ldc=N + 3, offset=offset)
    assert np.array_equal(c.astype(np.float64), oracle.reference(af, bf)[0])
    ab, bb, af, bf = operands(kind, M, N, K, "uniform", 2000 + K)
    cref, den = oracle.reference(af, bf)
    c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=lda, ldb=ldb, offset=offset)
    assert oracle.normalised_error(c, cref, den) <= TOL


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("N", [250, 260, 262, 301])
def test_mixed_moved_tiles_with_aligned_pitch(kind, N, variant, torch_gpu):
    """ldb a multiple of 8 elements (16-byte rows) with N not a multiple of
    8: an edge tile moved back to end at N starts its B columns at N - BN,
    so the copies of B must be narrower than 16 bytes (4-byte copies for an
    even N, 2-byte loads for an odd one).  Bit for bit on integer inputs."""
    M, K = 300, 100
    lda, ldb = K + (-K) % 8, N + (-N) % 8 + 8
    ab, bb, af, bf = operands(kind, M, N, K, "integer", 2100 + N)
    c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=lda, ldb=ldb, ldc=N + 1)
    assert np.array_equal(c.astype(np.float64), oracle.reference(af, bf)[0])


TWO_BYTE_SHAPES = [(256, 256, 1), (300, 260, 15), (257, 300, 32), (300, 257, 33), (520, 300, 64), (300, 520, 65),
                   (256, 512, 100), (513, 257, 1000)]


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("shape", TWO_BYTE_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in TWO_BYTE_SHAPES])
def test_mixed_two_byte_rows(kind, shape, variant, torch_gpu):
    """Rows only 2-byte aligned (odd leading dimensions, bases shifted by
    one element), M and N at least one large tile, so the raw 4-byte copies
    realigned in LDS run for the interior and moved edge tiles: K of one
    partial tile, one whole tile, a whole tile and a ragged one, many tiles.
    Bit for bit on integer inputs (each row's shift must be right), within
    the bar on uniform ones; NaN in every ld gap and around C."""
    M, N, K = shape
    ab, bb, af, bf = operands(kind, M, N, K, "integer", 2300 + M + N + K)
    want = oracle.reference(af, bf)[0]
    for lda, ldb, offset in ((K + 1, N + 1, 0), (K + 3, N + 5, 1), (K + 1, N + 2, 1), (K + 2, N + 1, 0)):
        c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=lda, ldb=ldb, ldc=N + 3, offset=offset)
        assert np.array_equal(c.astype(np.float64), want), (lda, ldb, offset)
    ab, bb, af, bf = operands(kind, M, N, K, "uniform", 2400 + M + N + K)
    cref, den = oracle.reference(af, bf)
    c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=K + 1, ldb=N + 1, offset=1)
    assert oracle.normalised_error(c, cref, den) <= TOL


_random_refs: dict = {}


@pytest.mark.parametrize("variant", VARIANTS, ids=VARIANT_IDS)
def test_mixed_random_shapes(variant, torch_gpu):
    """30 seeded random shapes (bf16), each with random leading-dimension
    pads and a base offset of 0, 1 or 2 elements, so that calls take the
    16-byte copies, the 4-byte copies or the 2-byte loads."""
    rng = np.random.default_rng(4242)
    for i in range(30):
        M, N, K = (int(x) for x in rng.integers(1, 600, 3))
        pa, pb, pc = (int(x) for x in rng.integers(0, 9, 3))
        offset = int(rng.integers(0, 3))
        if i not in _random_refs:
            ab, bb, af, bf = operands("bf16", M, N, K, "uniform", 6000 + i)
            _random_refs[i] = (ab, bb) + oracle.reference(af, bf)
        ab, bb, cref, den = _random_refs[i]
        c = run_mixed(torch_gpu, "bf16", ab, bb, variant, lda=K + pa, ldb=N + pb, ldc=N + pc, offset=offset)
        err = oracle.normalised_error(c, cref, den)
        assert err <= TOL, (M, N, K, pa, pb, pc, offset, err)


KSPLIT_VARIANTS = [dft.MIXED_64x64_KS2, dft.MIXED_64x64_KS4, dft.MIXED_32x64_KS4]


@pytest.mark.parametrize("kind", list(TYPES))
@pytest.mark.parametrize("K", [8, 64, 120, 128, 192, 200, 256, 320, 1000, 4100])
@pytest.mark.parametrize("variant", KSPLIT_VARIANTS, ids=[dft.MIXED_NAMES[v] for v in KSPLIT_VARIANTS])
def test_mixed_k_split_in_the_workgroup(kind, K, variant, torch_gpu):
    """K tiles of 64 dealt to 2 or 4 groups of waves: fewer tiles than
    groups, counts not a multiple of the groups, a ragged last tile in any
    group; partial sums added in LDS.  130 x 100 spans interior and moved
    edge tiles; bit for bit on integer operands."""
    M, N = 130, 104
    ab, bb, af, bf = operands(kind, M, N, K, "integer", 1700 + K)
    c = run_mixed(torch_gpu, kind, ab, bb, variant, lda=K + (8 - K % 8) % 8 + 8, ldb=N + 8, ldc=N + 3)
    assert np.array_equal(c.astype(np.float64), oracle.reference(af, bf)[0])
    ab, bb, af, bf = operands(kind, M, N, K, "uniform", 1800 + K)
    cref, den = oracle.reference(af, bf)
    assert oracle.normalised_error(run_mixed(torch_gpu, kind, ab, bb, variant), cref, den) <= TOL


@pytest.mark.parametrize("kind", list(TYPES))
def test_mixed_k_zero_and_empty(kind, torch_gpu):
    torch = torch_gpu
    c = torch.full((7, 9), float("nan"), device="cuda")
    st = dft.gemm_mixed_f32(TYPES[kind], 7, 9, 0, 0, 1, 0, 9, c.data_ptr(), 9, None, 0)
    torch.cuda.synchronize()
    assert st == dft.GEMM_OK and torch.all(c == 0)
    assert dft.gemm_mixed_f32(TYPES[kind], 0, 9, 5, 0, 5, 0, 9, 0, 9, None, 0) == dft.GEMM_OK


def test_matmul_mixed_wrapper(torch_gpu):
    torch = torch_gpu
    for dtype, kind in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        ab, bb, af, bf = operands(kind, 300, 260, 200, "uniform", 11)
        a = torch.from_numpy(ab.view(np.int16)).cuda().view(dtype)
        b = torch.from_numpy(bb.view(np.int16)).cuda().view(dtype)
        c = dft.matmul_mixed(a, b).cpu().numpy()
        cref, den = oracle.reference(af, bf)
        assert oracle.normalised_error(c, cref, den) <= TOL
    with pytest.raises(TypeError):
        dft.matmul_mixed(torch.zeros(4, 4, device="cuda"), torch.zeros(4, 4, device="cuda"))
