import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def golden_lines(name):
    """Non-comment, non-empty lines of a golden fixture file."""
    with open(os.path.join(GOLDEN, name)) as fh:
        return [ln.split() for ln in fh if ln.strip() and not ln.lstrip().startswith("#")]
