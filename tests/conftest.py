import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-side check")


def pytest_sessionstart(session):
    """Build the HIP library in-tree when it is missing (a fresh checkout);
    an existing build is used as is."""
    lib = os.path.join(ROOT, "dense_tiled_gemm_fp8_amd", "libgemm355.so")
    if not os.path.exists(lib):
        from dense_tiled_gemm_fp8_amd import build
        build.build()


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import reference
    if not os.path.exists(reference._LIB_PATH):
        reference.build(force=False)
    return reference
