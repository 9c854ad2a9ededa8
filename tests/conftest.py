import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key = value' lines, '#' comments."""
    vals = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (t.strip() for t in line.split("=", 1))
            vals[k] = float(v)
    return vals


@pytest.fixture
def golden():
    return read_golden
