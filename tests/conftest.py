"""Shared test set-up.  ``gpu`` marks tests that need an MI355X; everything
else runs on the CPU."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (runs the HIP library)")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle

    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build(force=True)
    yield
