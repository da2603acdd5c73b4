import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "fullsize: GPU parity at a full workload size")


def pytest_collection_modifyitems(config, items):
    """Run GPU tests in file order but put the full-size ones after the others,
    so a quick failure surfaces before the long cases, and the test of the
    allocation-free entry point last of all."""
    def rank(it):
        if it.module is not None and it.module.__name__.endswith("test_zz_no_alloc"):
            return 2
        return 1 if it.get_closest_marker("fullsize") else 0
    items.sort(key=rank)
