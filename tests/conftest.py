import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP kernels")
    config.addinivalue_line("markers", "slow: large inputs; minutes of host time")


def pytest_runtest_setup(item):
    # Name a GPU case on the real stderr before it runs, so a run that dies
    # inside a GPU call still shows which case it was in.
    if item.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[start] {item.nodeid}\n")
        sys.__stderr__.flush()
