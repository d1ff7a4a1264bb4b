import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


@pytest.fixture(scope="session")
def gemm_lib():
    """The HIP library (built in-tree if it is not there yet)."""
    import dense_fp32_tiled_amd as dft
    from dense_fp32_tiled_amd import build, lds_probe
    if not all(p.exists() for p in (dft.LIB_PATH, build.POISON_LIB, lds_probe.PROBE_LIB)):
        build.build_all()
    return dft.library()
