"""Pins for the fp64 CPU oracle: checks against facts fixed by the mathematics,
not against the oracle's own formula.

Each pin is a function ``pin(ref) -> None`` that raises AssertionError on a
mismatch, where ``ref(a, b, rows=None, cols=None, threads=None)`` returns
(C, Den) like ``oracle.reference``.  The same battery runs against the real
oracle (all must pass) and against copies of the oracle with a planted mistake
(at least one must fail), see test_oracle.py.

Coverage, by the mistake each one catches:
  hand_products      transposed operand, swapped index, wrong sign (hand-worked)
  identity           lda/ldb misuse, row/column offset errors on ragged shapes
  permutation        index mix-ups between rows and columns
  zero / k_zero      accumulator initialisation, K == 0 (empty sum)
  closed_forms       dropped first or last term (sum of 0..K-1), K == 1
  integer_exact      any dropped or duplicated term, at tile-scale shapes, vs
                     an int64 library product (exact)
  float_bound        fp64 accuracy: within gamma_K * Den of a library product
  brute_force        exact rational sums on every shape in {1..6}^3
  den                Den is the sum of |a||b| (exact on integer inputs)
  transpose          (AB)^T == B^T A^T bit for bit (same exact products, same order)
  k_split            AB == A1 B1 + A2 B2 exactly on integer inputs
  pitch              leading dimensions larger than the width; NaN in the gaps
                     is never read
  sampling           sampled rows/columns equal the full result bit for bit;
                     the result does not depend on the thread count
"""

from __future__ import annotations

import json
from fractions import Fraction
from pathlib import Path

import numpy as np

from workloads import draw, embed, make_operands

GOLDEN = Path(__file__).resolve().parent / "golden"
U = 2.0 ** -53  # unit roundoff of fp64


def gamma(k: int) -> float:
    return k * U / (1 - k * U)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def pin_hand_products(ref):
    cases = json.loads((GOLDEN / "hand_products.json").read_text())["cases"]
    for case in cases:
        c, d = ref(_f32(case["a"]), _f32(case["b"]))
        expect = np.asarray(case["c"], dtype=np.float64)
        assert c.shape == expect.shape, case["name"]
        assert np.array_equal(c, expect), (case["name"], c, expect)


def pin_identity(ref):
    for (M, K, seed) in [(7, 5, 1), (33, 17, 2), (130, 65, 3)]:
        rng = np.random.default_rng(seed)
        a = draw(rng, (M, K), "uniform")
        c, _ = ref(a, np.eye(K, dtype=np.float32))
        assert np.array_equal(c, a.astype(np.float64)), "A @ I != A"
        c, _ = ref(np.eye(M, dtype=np.float32), a)
        assert np.array_equal(c, a.astype(np.float64)), "I @ B != B"


def pin_permutation(ref):
    rng = np.random.default_rng(11)
    M, K, N = 9, 6, 11
    a = draw(rng, (M, K), "normal")
    b = draw(rng, (K, N), "normal")
    pk = rng.permutation(K)
    pm = rng.permutation(M)
    P = np.zeros((M, M), np.float32)
    P[np.arange(M), pm] = 1.0  # (P @ a)[i] = a[pm[i]]
    c, _ = ref(P, a)
    assert np.array_equal(c, a[pm].astype(np.float64)), "P @ A must permute rows"
    Q = np.zeros((K, K), np.float32)
    Q[pk, np.arange(K)] = 1.0  # (a @ Q)[:, j] = a[:, pk[j]]
    c, _ = ref(a, Q)
    assert np.array_equal(c, a[:, pk].astype(np.float64)), "A @ Q must permute columns"
    _ = b


def pin_zero(ref):
    rng = np.random.default_rng(5)
    a = draw(rng, (6, 4), "normal")
    b = draw(rng, (4, 3), "normal")
    c, d = ref(a, np.zeros((4, 3), np.float32))
    assert np.array_equal(c, np.zeros((6, 3))) and np.array_equal(d, np.zeros((6, 3)))
    c, d = ref(np.zeros((6, 4), np.float32), b)
    assert np.array_equal(c, np.zeros((6, 3)))


def pin_k_zero(ref):
    c, d = ref(np.zeros((3, 0), np.float32), np.zeros((0, 5), np.float32))
    assert c.shape == (3, 5)
    assert np.array_equal(c, np.zeros((3, 5))) and np.array_equal(d, np.zeros((3, 5)))


def pin_closed_forms(ref):
    for K in (1, 2, 16, 17, 513):
        c, d = ref(np.ones((3, K), np.float32), np.ones((K, 4), np.float32))
        assert np.array_equal(c, np.full((3, 4), float(K))), ("ones", K)
        assert np.array_equal(d, np.full((3, 4), float(K)))
        # A = 1, B[k][j] = k  ->  sum_{k<K} k = K(K-1)/2 (catches a dropped first or last term)
        b = np.repeat(np.arange(K, dtype=np.float32)[:, None], 4, axis=1)
        c, _ = ref(np.ones((3, K), np.float32), b)
        assert np.array_equal(c, np.full((3, 4), K * (K - 1) / 2.0)), ("triangular", K)
        # B[k][j] = k + 1 -> K(K+1)/2: the last term carries the largest weight
        c, _ = ref(np.ones((2, K), np.float32), b + 1)
        assert np.array_equal(c, np.full((2, 4), K * (K + 1) / 2.0)), ("triangular+1", K)
    # K == 1: rank-1 outer product, exact in fp64
    rng = np.random.default_rng(3)
    a = draw(rng, (5, 1), "normal")
    b = draw(rng, (1, 7), "normal")
    c, _ = ref(a, b)
    assert np.array_equal(c, a.astype(np.float64) * b.astype(np.float64))


def pin_integer_exact(ref):
    # Integer entries in [-4, 4]: every partial sum is an integer far below 2^53,
    # so the oracle must equal the exact int64 product bit for bit.
    for (M, N, K, seed) in [(37, 41, 129, 1), (128, 128, 128, 2), (100, 99, 513, 3), (5, 3, 4097, 4)]:
        a, b = make_operands(M, N, K, "integer", seed)
        c, d = ref(a, b)
        exact = a.astype(np.int64) @ b.astype(np.int64)
        assert np.array_equal(c, exact.astype(np.float64)), ("integer product", M, N, K)
        den = np.abs(a).astype(np.int64) @ np.abs(b).astype(np.int64)
        assert np.array_equal(d, den.astype(np.float64)), ("integer Den", M, N, K)


def pin_float_bound(ref):
    for (M, N, K, dist, seed) in [(31, 29, 257, "uniform", 7), (16, 20, 1000, "normal", 8)]:
        a, b = make_operands(M, N, K, dist, seed)
        c, d = ref(a, b)
        lib = a.astype(np.float64) @ b.astype(np.float64)
        # both sides are fp64 sums of the same exact products: each within gamma_K*Den of the truth
        assert np.all(np.abs(c - lib) <= 2 * gamma(K) * d + 1e-300), ("float bound", M, N, K)


def pin_brute_force(ref):
    rng = np.random.default_rng(99)
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                a = draw(rng, (M, K), "normal")
                b = draw(rng, (K, N), "uniform")
                c, d = ref(a, b)
                af = [[Fraction(float(x)) for x in row] for row in a]
                bf = [[Fraction(float(x)) for x in row] for row in b]
                for i in range(M):
                    for j in range(N):
                        exact = sum(af[i][k] * bf[k][j] for k in range(K))
                        den = sum(abs(af[i][k]) * abs(bf[k][j]) for k in range(K))
                        err = abs(Fraction(float(c[i, j])) - exact)
                        assert err <= Fraction(gamma(K)) * den, ("brute force", M, N, K, i, j)
                        derr = abs(Fraction(float(d[i, j])) - den)
                        assert derr <= Fraction(gamma(K)) * den, ("brute force Den", M, N, K, i, j)


def pin_transpose(ref):
    a, b = make_operands(23, 19, 37, "normal", 21)
    c, _ = ref(a, b)
    ct, _ = ref(np.ascontiguousarray(b.T), np.ascontiguousarray(a.T))
    assert np.array_equal(c.T, ct), "(AB)^T must equal B^T A^T bit for bit"


def pin_k_split(ref):
    a, b = make_operands(21, 26, 77, "integer", 31)
    c, _ = ref(a, b)
    for k1 in (1, 16, 30, 76):
        c1, _ = ref(np.ascontiguousarray(a[:, :k1]), np.ascontiguousarray(b[:k1]))
        c2, _ = ref(np.ascontiguousarray(a[:, k1:]), np.ascontiguousarray(b[k1:]))
        assert np.array_equal(c, c1 + c2), ("k split", k1)


def pin_pitch(ref):
    M, N, K = 13, 10, 9
    a, b = make_operands(M, N, K, "uniform", 41)
    c0, d0 = ref(a, b)
    for lda, ldb in [(K + 3, N), (K, N + 5), (K + 7, N + 1)]:
        abuf = embed(a, lda).reshape(M, lda)[:, :K]
        bbuf = embed(b, ldb).reshape(K, ldb)[:, :N]
        c, d = ref(abuf, bbuf)
        assert np.array_equal(c, c0) and np.array_equal(d, d0), ("pitch", lda, ldb)
        rows = np.array([0, 5, M - 1])
        cr, _ = ref(abuf, bbuf, rows=rows)
        assert np.array_equal(cr, c0[rows]), ("pitch rows", lda, ldb)
        cols = np.array([0, 4, N - 1])
        cc, _ = ref(abuf, bbuf, cols=cols)
        assert np.array_equal(cc, c0[:, cols]), ("pitch cols", lda, ldb)


def pin_sampling(ref):
    M, N, K = 40, 33, 65
    a, b = make_operands(M, N, K, "normal", 51)
    c, d = ref(a, b, threads=1)
    c7, d7 = ref(a, b, threads=7)
    assert np.array_equal(c, c7) and np.array_equal(d, d7), "thread count changed the result"
    rows = np.array([0, 3, 17, M - 1])
    cols = np.array([0, 1, 20, N - 1])
    cr, dr = ref(a, b, rows=rows, threads=3)
    cc, dc = ref(a, b, cols=cols, threads=5)
    assert np.array_equal(cr, c[rows]) and np.array_equal(dr, d[rows])
    assert np.array_equal(cc, c[:, cols]) and np.array_equal(dc, d[:, cols])


PINS = {
    "hand_products": pin_hand_products,
    "identity": pin_identity,
    "permutation": pin_permutation,
    "zero": pin_zero,
    "k_zero": pin_k_zero,
    "closed_forms": pin_closed_forms,
    "integer_exact": pin_integer_exact,
    "float_bound": pin_float_bound,
    "brute_force": pin_brute_force,
    "transpose": pin_transpose,
    "k_split": pin_k_split,
    "pitch": pin_pitch,
    "sampling": pin_sampling,
}


def run_battery(ref, skip=()) -> dict[str, str]:
    """Run every pin; return {name: failure message} for those that fail."""
    failures = {}
    for name, pin in PINS.items():
        if name in skip:
            continue
        try:
            pin(ref)
        except Exception as e:  # noqa: BLE001 - a crash in a mutant is a detection too
            failures[name] = f"{type(e).__name__}: {e}"[:200]
    return failures
