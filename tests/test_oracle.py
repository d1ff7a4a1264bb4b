"""The fp64 CPU oracle against its pins, and planted mistakes against the pins.

The oracle is the reference for every parity test of the GPU path, so it is
checked here against facts the mathematics fixes (see oracle_pins.py), and a
copy of it with a planted mistake must fail at least one of those checks.
"""

from __future__ import annotations

import subprocess

import numpy as np
import pytest

import oracle
from oracle_pins import PINS, run_battery


@pytest.mark.parametrize("name", sorted(PINS))
def test_oracle_pin(name, oracle_lib):
    PINS[name](lambda a, b, **kw: oracle.reference(a, b, lib=oracle_lib, **kw))


def test_normalised_error_rules():
    cref = np.array([[1.0, 0.0], [2.0, -3.0]])
    den = np.array([[2.0, 0.0], [4.0, 6.0]])
    assert oracle.normalised_error(cref.copy(), cref, den) == 0.0
    c = cref.copy()
    c[1, 1] += 0.6  # 0.6 / 6
    assert oracle.normalised_error(c, cref, den) == pytest.approx(0.1)
    c = cref.copy()
    c[0, 1] = 1e-30  # Den == 0 demands an exact match
    assert oracle.normalised_error(c, cref, den) == float("inf")
    c = cref.copy()
    c[0, 0] = np.nan
    assert oracle.normalised_error(c, cref, den) == float("inf")


def test_rejects_bad_arguments(oracle_lib):
    a = np.zeros((2, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.reference(a, np.zeros((4, 2), np.float32), lib=oracle_lib)
    with pytest.raises(RuntimeError):
        oracle.reference(a, np.zeros((3, 2), np.float32), rows=[2], lib=oracle_lib)
    with pytest.raises(RuntimeError):
        oracle.reference(a, np.zeros((3, 2), np.float32), cols=[-1], lib=oracle_lib)


# (description, text in oracle_gemm.c, replacement, occurrence to replace)
MUTANTS = [
    ("drop the last k term", "for (int64_t k = 0; k < job->K; ++k) {\n            const double a = (double)arow[k];\n            const double abs_a",
     "for (int64_t k = 0; k + 1 < job->K; ++k) {\n            const double a = (double)arow[k];\n            const double abs_a"),
    ("drop the first k term", "for (int64_t k = 0; k < job->K; ++k) {\n            const double a = (double)arow[k];\n            const double abs_a",
     "for (int64_t k = 1; k < job->K; ++k) {\n            const double a = (double)arow[k];\n            const double abs_a"),
    ("wrong sign", "c[j] += a * b;", "c[j] -= a * b;"),
    ("A indexed without its row pitch", "const float *arow = job->A + i * job->lda;\n        for (int64_t k",
     "const float *arow = job->A + i;\n        for (int64_t k"),
    ("B indexed without its row pitch", "const float *brow = job->B + k * job->ldb;",
     "const float *brow = job->B + k;"),
    ("lda taken as K", "const float *arow = job->A + i * job->lda;\n        for (int64_t k",
     "const float *arow = job->A + i * job->K;\n        for (int64_t k"),
    ("ldb taken as N", "const float *brow = job->B + k * job->ldb;", "const float *brow = job->B + k * job->N;"),
    ("Den without absolute values", "d[j] += abs_a * fabs(b);", "d[j] += a * b;"),
    ("accumulate in fp32", "c[j] += a * b;", "c[j] = (float)(c[j] + a * b);"),
    ("column gather uses the position, not the column index", "bcols[c * K + k] = (double)B[k * ldb + cols[c]];",
     "bcols[c * K + k] = (double)B[k * ldb + c];"),
    ("selected row ignored", "const int64_t i = job->rows[r];", "const int64_t i = r;"),
    ("transposed A in the column path", "const float *arow = job->A + i * job->lda;\n        for (int64_t c",
     "const float *arow = job->A + i;\n        for (int64_t c"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new, tmp_path):
    src = oracle._SRC.read_text()
    assert src.count(old) == 1, f"mutation site not unique for {desc!r}"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib_path = oracle.build(mutant_src, tmp_path / "libmutant.so")
    lib = oracle.load(lib_path)
    failures = run_battery(lambda a, b, **kw: oracle.reference(a, b, lib=lib, **kw),
                           skip=("brute_force",))
    assert failures, f"no pin caught the planted mistake: {desc}"


def test_oracle_builds_warning_free(tmp_path):
    out = subprocess.run(["gcc", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared", "-pthread",
                          str(oracle._SRC), "-o", str(tmp_path / "lib.so"), "-lm"],
                         capture_output=True, text=True)
    assert out.returncode == 0, out.stderr


def test_config1_single_thread_is_well_under_a_second(oracle_lib):
    """The 128^3 product on one host thread: the oracle's own speed bar (best
    of three runs, so a busy host does not fail it)."""
    import time

    import workloads

    cfg = workloads.CONFIG_BY_NAME["small128"]
    a, b = workloads.config_operands(cfg)
    best = float("inf")
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.reference(a, b, threads=1, lib=oracle_lib)
        best = min(best, time.perf_counter() - t0)
    assert best < 0.5, best
