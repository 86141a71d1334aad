import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (1 GiB index-K)")


def pytest_runtest_setup(item):
    # Name each test before it runs, so a GPU run that dies still says which case it was in.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[case] {item.nodeid}", flush=True)
