import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    # On a host with no GPU driver node at all, GPU tests are skipped so that a
    # plain `pytest tests/` works there.  Where /dev/kfd exists they always run
    # and fail loudly if the device or the HIP library is unusable.
    if os.path.exists("/dev/kfd"):
        return
    skip = pytest.mark.skip(reason="no GPU driver on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
