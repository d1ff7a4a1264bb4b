"""Python binding for the gfx950 masked, LDS-tiled fp32 GEMM.

Argument marshalling only: every function below forwards to the entry point of
the same name in libdense_fp32_tiled.so (declared in include/dense_fp32_tiled.h)
through ctypes.  ``matmul`` is a convenience wrapper that takes torch tensors,
passes their device pointers, row pitches and the current HIP stream, and
raises GemmError on a non-zero status.  There is no fallback: if the HIP
library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
LIB_PATH = PKG_DIR / "libdense_fp32_tiled.so"

GEMM_OK = 0
GEMM_ERR_INVALID_DIM = -1
GEMM_ERR_INVALID_LD = -2
GEMM_ERR_NULL = -3
GEMM_ERR_ALIAS = -4
GEMM_ERR_UNSUPPORTED = -5
GEMM_ERR_CONFIG = -6
GEMM_ERR_HIP = -7
GEMM_ERR_TOO_LARGE = -8
GEMM_ERR_WORKSPACE = -9
GEMM_ERR_SCRATCH = -10

VARIANT_AUTO = 0
VARIANT_MFMA = 1
VARIANT_VALU = 2
VARIANT_MFMA_STAGES1 = 3
VARIANT_MFMA_NOPAD = 4
VARIANT_MFMA_SCALAR = 5
VARIANT_MFMA16 = 6
VARIANT_MFMA_128 = 7
VARIANT_MFMA_128_BK32 = 8
VARIANT_MFMA_DIRECT = 9
VARIANT_MFMA_128_DIRECT = 10
VARIANT_MFMA_128_BK32_DIRECT = 11
VARIANT_MFMA_64_DIRECT = 12
VARIANT_MFMA_256x256_DIRECT = 13
VARIANT_MFMA_256x256_W4_DIRECT = 14
VARIANT_MFMA_256x256_PIPE = 15
VARIANT_MFMA_256x256_BK32_PIPE = 16
VARIANT_MFMA16_256x256_DIRECT = 17
VARIANT_MFMA16_256x256_W4_BK32_PIPE = 18
VARIANT_MFMA_64_BK32_DIRECT = 19
VARIANT_MFMA_64_KS4 = 20
VARIANT_MFMA_32x64_KS4 = 21
VARIANT_MFMA_32x32_KS8 = 22
VARIANT_MFMA_64_BK32_PIPE = 23
VARIANT_MFMA_64_KS2 = 24
VARIANT_COUNT = 25
# 16-bit inputs with fp32 accumulation (gemm_mixed_f32)
INPUT_BF16 = 0
INPUT_F16 = 1
INPUT_NAMES = {INPUT_BF16: "bf16", INPUT_F16: "f16"}
MIXED_AUTO = 0
MIXED_256x128 = 1
MIXED_256x256 = 2
MIXED_256x128_BK64 = 3
MIXED_128x128_BK64 = 4
MIXED_256x256_S3 = 5
MIXED_256x256_BK64 = 6
MIXED_64x64 = 7
MIXED_64x64_KS2 = 8
MIXED_64x64_KS4 = 9
MIXED_32x64_KS4 = 10
MIXED_COUNT = 11
MIXED_NAMES = {MIXED_AUTO: "auto", MIXED_256x128: "256x128", MIXED_256x256: "256x256",
               MIXED_256x128_BK64: "256x128_bk64", MIXED_128x128_BK64: "128x128_bk64", MIXED_256x256_S3: "256x256_s3",
               MIXED_256x256_BK64: "256x256_bk64", MIXED_64x64: "64x64", MIXED_64x64_KS2: "64x64_ks2",
               MIXED_64x64_KS4: "64x64_ks4", MIXED_32x64_KS4: "32x64_ks4"}
VARIANT_NAMES = {
    VARIANT_AUTO: "auto",
    VARIANT_MFMA: "mfma",
    VARIANT_VALU: "valu",
    VARIANT_MFMA_STAGES1: "mfma_stages1",
    VARIANT_MFMA_NOPAD: "mfma_nopad",
    VARIANT_MFMA_SCALAR: "mfma_scalar",
    VARIANT_MFMA16: "mfma16",
    VARIANT_MFMA_128: "mfma_128",
    VARIANT_MFMA_128_BK32: "mfma_128_bk32",
    VARIANT_MFMA_DIRECT: "mfma_direct",
    VARIANT_MFMA_128_DIRECT: "mfma_128_direct",
    VARIANT_MFMA_128_BK32_DIRECT: "mfma_128_bk32_direct",
    VARIANT_MFMA_64_DIRECT: "mfma_64_direct",
    VARIANT_MFMA_256x256_DIRECT: "mfma_256x256_direct",
    VARIANT_MFMA_256x256_W4_DIRECT: "mfma_256x256_w4_direct",
    VARIANT_MFMA_256x256_PIPE: "mfma_256x256_pipe",
    VARIANT_MFMA_256x256_BK32_PIPE: "mfma_256x256_bk32_pipe",
    VARIANT_MFMA16_256x256_DIRECT: "mfma16_256x256_direct",
    VARIANT_MFMA16_256x256_W4_BK32_PIPE: "mfma16_256x256_w4_bk32_pipe",
    VARIANT_MFMA_64_BK32_DIRECT: "mfma_64_bk32_direct",
    VARIANT_MFMA_64_KS4: "mfma_64_ks4",
    VARIANT_MFMA_32x64_KS4: "mfma_32x64_ks4",
    VARIANT_MFMA_32x32_KS8: "mfma_32x32_ks8",
    VARIANT_MFMA_64_BK32_PIPE: "mfma_64_bk32_pipe",
    VARIANT_MFMA_64_KS2: "mfma_64_ks2",
}

# Every symbol the public header declares.
EXPORTS = (
    "gemm_f32",
    "gemm_f32_ex",
    "gemm_f32_tile_config",
    "gemm_f32_status_string",
    "gemm_f32_splitk",
    "gemm_f32_splitk_ex",
    "gemm_f32_splitk_noalloc",
    "gemm_f32_splitk_auto_variant",
    "gemm_f32_splitk_workspace_bytes",
    "gemm_f32_splitk_auto_splits",
    "gemm_f32_auto_variant",
    "gemm_f32_auto_variant_ex",
    "gemm_mixed_f32",
    "gemm_mixed_tile_config",
    "gemm_mixed_auto_variant",
    "gemm_lds_choose_mfma_layout",
    "gemm_lds_layout",
    "gemm_lds_offset",
    "gemm_lds_bank",
    "gemm_lds_conflict_degree",
    "gemm_lds_access_cycles",
    "gemm_lds_page_pad",
)


class GemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = gemm_f32_status_string(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


class TileConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "variant", "bm", "bn", "bk", "threads", "wave_size", "tm", "tn", "stages", "barriers_per_tile",
        "a_rows", "a_cols", "a_pad", "a_row_stride", "a_stage_elems",
        "b_rows", "b_cols", "b_pad", "b_row_stride", "b_stage_elems",
        "lds_bytes", "vec_width", "lds_banks_b32", "lds_lanes_b32", "lds_banks_b128", "lds_lanes_b128",
        "a_transposed", "a_swz_unit", "a_swz_shift", "a_swz_mask", "b_swz_unit", "b_swz_shift", "b_swz_mask",
        "mfma_block", "xcd_tile_order", "direct_to_lds", "elem_bytes", "k_groups")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def _share_torch_hip_runtime():
    """Load torch (if installed) before the HIP library.  torch ships its own
    HIP runtime with the same soname (libamdhip64.so.7) as ROCm's; loaded
    first, it satisfies this library's dependency, so both share one runtime
    and torch's streams and allocations are valid here.  Loaded the other way
    round, the process would hold two runtimes and torch's stream handles
    would be rejected by this library's launches."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def library(path: Path | None = None):
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is not built; run `python -m dense_fp32_tiled_amd.build`")
    _share_torch_hip_runtime()
    lib = ctypes.CDLL(str(p))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    gemm_args = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.gemm_f32.argtypes = gemm_args
    lib.gemm_f32.restype = ctypes.c_int
    lib.gemm_f32_ex.argtypes = gemm_args + [ctypes.c_int]
    lib.gemm_f32_ex.restype = ctypes.c_int
    lib.gemm_f32_tile_config.argtypes = [ctypes.c_int, ctypes.POINTER(TileConfig)]
    lib.gemm_f32_tile_config.restype = ctypes.c_int
    lib.gemm_f32_status_string.argtypes = [ctypes.c_int]
    lib.gemm_f32_status_string.restype = ctypes.c_char_p
    lib.gemm_f32_splitk.argtypes = gemm_args[:9] + [vp, i64, ctypes.c_int, vp]
    lib.gemm_f32_splitk.restype = ctypes.c_int
    lib.gemm_f32_splitk_ex.argtypes = gemm_args[:9] + [vp, i64, ctypes.c_int, vp, ctypes.c_int]
    lib.gemm_f32_splitk_ex.restype = ctypes.c_int
    lib.gemm_f32_splitk_noalloc.argtypes = gemm_args[:9] + [ctypes.c_int, vp]
    lib.gemm_f32_splitk_noalloc.restype = ctypes.c_int
    lib.gemm_f32_splitk_auto_variant.argtypes = []
    lib.gemm_f32_splitk_auto_variant.restype = ctypes.c_int
    lib.gemm_f32_splitk_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int, i32]
    lib.gemm_f32_splitk_workspace_bytes.restype = i64
    lib.gemm_f32_splitk_auto_splits.argtypes = [i64, i64, i64, i32]
    lib.gemm_f32_splitk_auto_splits.restype = ctypes.c_int
    lib.gemm_f32_auto_variant.argtypes = [i64, i64, i64, i32]
    lib.gemm_f32_auto_variant.restype = ctypes.c_int
    lib.gemm_f32_auto_variant_ex.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.gemm_f32_auto_variant_ex.restype = ctypes.c_int
    lib.gemm_mixed_f32.argtypes = [ctypes.c_int] + gemm_args[:9] + [vp, ctypes.c_int]
    lib.gemm_mixed_f32.restype = ctypes.c_int
    lib.gemm_mixed_tile_config.argtypes = [ctypes.c_int, ctypes.POINTER(TileConfig)]
    lib.gemm_mixed_tile_config.restype = ctypes.c_int
    lib.gemm_mixed_auto_variant.argtypes = [i64, i64, i64, i32]
    lib.gemm_mixed_auto_variant.restype = ctypes.c_int
    lib.gemm_lds_choose_mfma_layout.argtypes = [i32] * 8 + [ctypes.POINTER(i32)]
    lib.gemm_lds_choose_mfma_layout.restype = ctypes.c_int
    p32 = ctypes.POINTER(i32)
    lib.gemm_lds_layout.argtypes = [i32, i32, i32, i32, p32, p32, p32, p32]
    lib.gemm_lds_layout.restype = ctypes.c_int
    lib.gemm_lds_offset.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.gemm_lds_offset.restype = i64
    lib.gemm_lds_bank.argtypes = [i64, i32]
    lib.gemm_lds_bank.restype = i32
    lib.gemm_lds_conflict_degree.argtypes = [ctypes.POINTER(i64), i32, i32, i32, i32]
    lib.gemm_lds_conflict_degree.restype = i32
    lib.gemm_lds_access_cycles.argtypes = [ctypes.POINTER(i64), i32]
    lib.gemm_lds_access_cycles.restype = i32
    lib.gemm_lds_page_pad.argtypes = [i32, i32, i32]
    lib.gemm_lds_page_pad.restype = i32
    if path is None:
        _lib = lib
    return lib


# ---- entry points, same names as the C ABI --------------------------------------
def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> int:
    return library().gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, stream=None, variant=VARIANT_AUTO) -> int:
    return library().gemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, variant)


def gemm_f32_tile_config(variant: int) -> dict:
    cfg = TileConfig()
    st = library().gemm_f32_tile_config(variant, ctypes.byref(cfg))
    if st != GEMM_OK:
        raise GemmError(st, f"gemm_f32_tile_config({variant})")
    return cfg.as_dict()


def gemm_f32_status_string(status: int) -> str:
    return library().gemm_f32_status_string(status).decode()


def gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, splits=0, stream=None) -> int:
    return library().gemm_f32_splitk(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, splits, stream)


def gemm_f32_splitk_ex(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, splits=0, stream=None,
                       variant=VARIANT_AUTO) -> int:
    return library().gemm_f32_splitk_ex(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, splits, stream,
                                        variant)


def gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, splits=0, stream=None) -> int:
    return library().gemm_f32_splitk_noalloc(M, N, K, A, lda, B, ldb, C, ldc, splits, stream)


def gemm_f32_splitk_auto_variant() -> int:
    return library().gemm_f32_splitk_auto_variant()


def gemm_f32_splitk_workspace_bytes(M: int, N: int, K: int, splits: int, num_cus: int) -> int:
    return library().gemm_f32_splitk_workspace_bytes(M, N, K, splits, num_cus)


def gemm_f32_splitk_auto_splits(M: int, N: int, K: int, num_cus: int) -> int:
    return library().gemm_f32_splitk_auto_splits(M, N, K, num_cus)


def gemm_f32_auto_variant(M: int, N: int, K: int, num_cus: int) -> int:
    return library().gemm_f32_auto_variant(M, N, K, num_cus)


def gemm_f32_auto_variant_ex(M: int, N: int, K: int, num_cus: int, a_rows_aligned: bool, b_rows_aligned: bool) -> int:
    return library().gemm_f32_auto_variant_ex(M, N, K, num_cus, int(a_rows_aligned), int(b_rows_aligned))


def gemm_mixed_f32(input_type, M, N, K, A, lda, B, ldb, C, ldc, stream=None, variant=MIXED_AUTO) -> int:
    return library().gemm_mixed_f32(input_type, M, N, K, A, lda, B, ldb, C, ldc, stream, variant)


def gemm_mixed_tile_config(variant: int) -> dict:
    cfg = TileConfig()
    st = library().gemm_mixed_tile_config(variant, ctypes.byref(cfg))
    if st != GEMM_OK:
        raise GemmError(st, "gemm_mixed_tile_config")
    return cfg.as_dict()


def gemm_mixed_auto_variant(M: int, N: int, K: int, num_cus: int) -> int:
    return library().gemm_mixed_auto_variant(M, N, K, num_cus)


def gemm_lds_choose_mfma_layout(bm, bn, bk, wm, wn, mb, vec, direct=0):
    """(status, (pad, unit, shift, mask) of A, (pad, unit, shift, mask) of B)."""
    out = (ctypes.c_int32 * 8)()
    st = library().gemm_lds_choose_mfma_layout(bm, bn, bk, wm, wn, mb, vec, direct, out)
    return st, tuple(out[:4]), tuple(out[4:])


def gemm_lds_layout(rows: int, cols: int, pad: int, stages: int):
    """(status, row_stride, stage_elems, total_elems, bytes)."""
    out = [ctypes.c_int32(-1) for _ in range(4)]
    st = library().gemm_lds_layout(rows, cols, pad, stages, *[ctypes.byref(x) for x in out])
    return (st, *[x.value for x in out])


def gemm_lds_offset(rows, cols, pad, stages, stage, row, col) -> int:
    return library().gemm_lds_offset(rows, cols, pad, stages, stage, row, col)


def gemm_lds_bank(word_offset: int, banks: int) -> int:
    return library().gemm_lds_bank(word_offset, banks)


def gemm_lds_conflict_degree(lane_words, width: int, banks: int, group: int) -> int:
    arr = (ctypes.c_int64 * len(lane_words))(*lane_words)
    return library().gemm_lds_conflict_degree(arr, len(lane_words), width, banks, group)


def gemm_lds_access_cycles(lane_words, mode: int) -> int:
    """LDS cycles of one 64-lane access under the gfx950 bank model (see the header)."""
    words = list(lane_words)
    if len(words) != 64:
        raise ValueError("64 lane offsets")
    return library().gemm_lds_access_cycles((ctypes.c_int64 * 64)(*words), mode)


def gemm_lds_page_pad(columns: int, simultaneous_rows: int, banks: int = 32) -> int:
    return library().gemm_lds_page_pad(columns, simultaneous_rows, banks)


# ---- torch convenience -------------------------------------------------------------
def _operand(t, name, dtype=None):
    """(device pointer, row pitch in elements) of a 2-D tensor whose rows are
    laid out one after another: unit column stride, and a row stride of at
    least the row length (a tensor whose rows overlap, e.g. an expanded
    view with row stride 0, has no such pitch and is rejected)."""
    import torch

    dtype = dtype or torch.float32
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D {dtype} tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    if rows > 1 and cols > 0 and t.stride(0) < cols:
        raise ValueError(f"{name} has overlapping rows (row stride {t.stride(0)} < {cols} columns)")
    ld = t.stride(0) if rows > 1 and cols > 0 else max(cols, 1)
    return t.data_ptr(), ld


def _operands(a, b, out, dtype=None, out_dtype=None):
    """Checks shared by the torch wrappers, all before any launch: operand
    types and layouts, matching inner dimensions, every tensor on a's device
    and `out` (allocated here when None) of shape (M, N).  Returns
    (M, N, K, (pa, lda), (pb, ldb), (pc, ldc), out)."""
    import torch

    pa, lda = _operand(a, "a", dtype)
    pb, ldb = _operand(b, "b", dtype)
    M, K = a.shape
    if b.shape[0] != K:
        raise ValueError(f"inner dimensions differ: {K} vs {b.shape[0]}")
    N = b.shape[1]
    if b.device != a.device:
        raise ValueError(f"b is on {b.device}, a on {a.device}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=a.device)
    elif tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    pc, ldc = _operand(out, "out", out_dtype)
    if out.device != a.device:
        raise ValueError(f"out is on {out.device}, a on {a.device}")
    return M, N, K, (pa, lda), (pb, ldb), (pc, ldc), out


def _stream_handle(stream, device):
    import torch

    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def matmul_splitk(a, b, out=None, splits: int = 0, workspace=None, stream=None, variant: int = VARIANT_AUTO):
    """C = a @ b with gemm_f32_splitk_ex (slices run by `variant`, AUTO = the
    library's split-K kernel).  The workspace (a float32 tensor on the same
    device) is allocated here when not given."""
    import torch

    M, N, K, (pa, lda), (pb, ldb), (pc, ldc), out = _operands(a, b, out)
    cus = torch.cuda.get_device_properties(a.device).multi_processor_count
    need = gemm_f32_splitk_workspace_bytes(M, N, K, splits, cus)
    if need < 0:
        raise GemmError(need, "gemm_f32_splitk_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=a.device)
    elif workspace is not None and workspace.device != a.device:
        raise ValueError(f"workspace is on {workspace.device}, a on {a.device}")
    wp = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(a.device):
        st = gemm_f32_splitk_ex(M, N, K, pa, lda, pb, ldb, pc, ldc, wp, wbytes, splits,
                                _stream_handle(stream, a.device), variant)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_f32_splitk_ex")
    return out


def matmul_mixed(a, b, out=None, variant: int = MIXED_AUTO, stream=None):
    """C (float32) = a @ b for bfloat16 or float16 tensors a (M x K) and b
    (K x N) of the same dtype, accumulated in fp32 by gemm_mixed_f32."""
    import torch

    types = {torch.bfloat16: INPUT_BF16, torch.float16: INPUT_F16}
    if a.dtype not in types or b.dtype != a.dtype:
        raise TypeError("a and b must both be bfloat16 or both float16")
    M, N, K, (pa, lda), (pb, ldb), (pc, ldc), out = _operands(a, b, out, a.dtype)
    with torch.cuda.device(a.device):
        st = gemm_mixed_f32(types[a.dtype], M, N, K, pa, lda, pb, ldb, pc, ldc, _stream_handle(stream, a.device),
                            variant)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_mixed_f32")
    return out


def matmul(a, b, out=None, variant: int = VARIANT_AUTO, stream=None):
    """C = a @ b on the GPU with the HIP kernels.  a: M x K, b: K x N, float32,
    unit column stride (row pitch may exceed the width).  Enqueued on `stream`
    (a torch.cuda.Stream or raw handle) or torch's current stream."""
    import torch

    M, N, K, (pa, lda), (pb, ldb), (pc, ldc), out = _operands(a, b, out)
    if stream is None:
        handle = torch.cuda.current_stream(a.device).cuda_stream
    elif isinstance(stream, int):
        handle = stream
    else:
        handle = stream.cuda_stream
    with torch.cuda.device(a.device):
        st = gemm_f32_ex(M, N, K, pa, lda, pb, ldb, pc, ldc, handle, variant)
    if st != GEMM_OK:
        raise GemmError(st, "gemm_f32_ex")
    return out
