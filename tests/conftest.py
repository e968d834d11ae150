import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU sweep; runs only with EP_RUN_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("EP_RUN_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow sweep: set EP_RUN_SLOW=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)
