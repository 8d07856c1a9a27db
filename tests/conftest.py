import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests print what they run before touching the device, so that a failure names its case.
    for it in items:
        if it.get_closest_marker("gpu") is not None:
            it.add_marker(pytest.mark.timeout(600))
