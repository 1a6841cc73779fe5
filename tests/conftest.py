import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long exhaustive CPU check; runs only with PURO_FP8_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("PURO_FP8_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive check; set PURO_FP8_SLOW=1 to run")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
