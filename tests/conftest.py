import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running host test")


def pytest_collection_modifyitems(config, items):
    # GPU tests that create large inputs run late so a failure in a small case shows first; the
    # static-workspace entry point's test runs last of all (after every other call has used the
    # GPU), as a stable sort keeps the rest in file order.
    def rank(it):
        name = it.module.__name__
        return 2 if name.endswith("test_zz_no_alloc") else (1 if name.endswith("test_gpu_full") else 0)
    items.sort(key=rank)
