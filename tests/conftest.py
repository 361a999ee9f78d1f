import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


def pytest_collection_modifyitems(config, items):
    """GPU tests are skipped, not failed, where no GPU is visible."""
    if not any(item.get_closest_marker("gpu") for item in items):
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if item.get_closest_marker("gpu"):
            item.add_marker(skip)


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Builds the CPU oracle if this checkout has not built it yet."""
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib):
        from oracle import build as ob
        ob.build()
    yield
