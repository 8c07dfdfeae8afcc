import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Put every GPU test after the CPU tests so that a round-end `-x` run reports
    # CPU failures first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)
