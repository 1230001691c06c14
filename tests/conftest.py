import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    # Files named test_gpu_* hold GPU parity tests; mark them even if a test
    # forgot the decorator, so the CPU run never touches them.
    for it in items:
        if os.path.basename(str(it.fspath)).startswith("test_gpu"):
            it.add_marker(pytest.mark.gpu)
