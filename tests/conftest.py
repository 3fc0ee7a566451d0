import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Integer matrix from a text fixture under tests/golden ('#' lines are comments)."""
    import numpy as np
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=np.int64)


@pytest.fixture(scope="session")
def golden():
    return load_golden
