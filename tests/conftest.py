import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload")


def pytest_collection_modifyitems(config, items):
    # Run the GPU tests in file order, but the full-size ones after the
    # small ones, so a failure on a small case shows first, and the
    # no-allocation entry point's test (test_zz_*) last of all.
    def rank(it):
        if os.path.basename(str(it.fspath)).startswith("test_zz_"):
            return 2
        return 1 if it.get_closest_marker("slow") else 0
    items.sort(key=rank)
