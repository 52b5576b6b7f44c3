import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built librr.so")
    config.addinivalue_line("markers", "slow: oracle runs that take more than a few seconds")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Rows of a whitespace-separated fixture; lines starting with '#' are comments."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows
