import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_setup(item):
    if "gpu" in item.keywords:
        # Print the case name before any GPU work starts, so a run that ends
        # the process still names the case that was running.
        sys.stderr.write(f"\n[gpu-case] {item.nodeid}\n")
        sys.stderr.flush()
