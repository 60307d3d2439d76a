import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long oracle run (minutes); runs only with GPT_RUN_SLOW=1")


def pytest_collection_modifyitems(config, items):
    import pytest
    if os.environ.get("GPT_RUN_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="long oracle run: set GPT_RUN_SLOW=1 to include it")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)
