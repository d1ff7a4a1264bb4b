"""fp64 CPU oracle for C = A @ B with fp32 operands.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code that may import this package.  The GPU
library never imports it, links it or calls it, and it imports nothing from
the GPU library.

The arithmetic lives in ``oracle_gemm.c`` (plain C, fp64 accumulation in
ascending k, see that file's header).  This module builds it with gcc, loads it
with ctypes and adds the normalised error used to compare a result with it:

    err = max_{i,j} |C[i][j] - Cref[i][j]| / Den[i][j],
    Den[i][j] = sum_k |A[i][k]| * |B[k][j]|

where an element with Den == 0 (every term is zero, e.g. K == 0) must equal
Cref exactly, else its ratio is infinite; a NaN in C also counts as infinite.
Den is the bound that standard floating-point error analysis of a sum of
products gives (the error of a length-K dot product is at most gamma_K * Den),
so the ratio is scale-free and does not blow up where C itself is near zero.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle_gemm.c"
_LIB = _HERE / "liboracle_gemm.so"
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-std=c11"]

_lib = None


def build(src: Path = _SRC, out: Path = _LIB) -> Path:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = out.with_suffix(".so.tmp")
    subprocess.run(["gcc", *_CFLAGS, str(src), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: Path | None = None):
    """Load the compiled oracle (building it first if it is not there)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(str(path)))
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        _lib = _bind(ctypes.CDLL(str(_LIB)))
    return _lib


def _bind(lib):
    i64, p = ctypes.c_int64, ctypes.c_void_p
    for name in ("oracle_gemm_rows", "oracle_gemm_cols"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p, p, ctypes.c_int]
    return lib


def host_threads() -> int:
    return len(os.sched_getaffinity(0))


def _operand(x: np.ndarray, name: str) -> tuple[np.ndarray, int]:
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return x, max(1, x.shape[1])
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    ld = x.strides[0] // 4 if x.shape[0] > 1 else max(1, x.shape[1])
    return x, max(ld, x.shape[1], 1)


def reference(a: np.ndarray, b: np.ndarray, rows=None, cols=None, threads: int | None = None,
              lib=None):
    """Oracle product of a (M x K) and b (K x N), both float32, row-major with
    unit column stride (a row pitch larger than the width is allowed).

    rows=None, cols=None: full M x N result.
    rows=idx: the selected rows (len(idx) x N).  cols=idx: the selected
    columns (M x len(idx)).  Returns (C, Den) as float64 arrays.
    """
    lib = lib or load()
    a, lda = _operand(a, "a")
    b, ldb = _operand(b, "b")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    threads = threads or host_threads()
    if rows is not None and cols is not None:
        raise ValueError("give rows or cols, not both")
    if cols is None:
        idx = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        c = np.empty((len(idx), N), dtype=np.float64)
        d = np.empty((len(idx), N), dtype=np.float64)
        rc = lib.oracle_gemm_rows(M, N, K, a.ctypes.data, lda, b.ctypes.data, ldb,
                                  idx.ctypes.data, len(idx), c.ctypes.data, d.ctypes.data, threads)
    else:
        idx = np.ascontiguousarray(cols, dtype=np.int64)
        c = np.empty((M, len(idx)), dtype=np.float64)
        d = np.empty((M, len(idx)), dtype=np.float64)
        rc = lib.oracle_gemm_cols(M, N, K, a.ctypes.data, lda, b.ctypes.data, ldb,
                                  idx.ctypes.data, len(idx), c.ctypes.data, d.ctypes.data, threads)
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return c, d


def normalised_error(c: np.ndarray, cref: np.ndarray, den: np.ndarray) -> float:
    """max |C - Cref| / Den in fp64; see the module docstring for Den == 0."""
    c = np.asarray(c, dtype=np.float64)
    if c.shape != cref.shape or c.shape != den.shape:
        raise ValueError("shape mismatch")
    if c.size == 0:
        return 0.0
    if not np.all(np.isfinite(c)):
        return float("inf")
    diff = np.abs(c - cref)
    zero = den == 0.0
    if np.any(diff[zero] != 0.0):
        return float("inf")
    ratio = np.zeros_like(diff)
    np.divide(diff, den, out=ratio, where=~zero)
    return float(ratio.max())
