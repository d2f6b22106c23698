import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


def golden(name):
    """Value of one closed-form constant from tests/golden/closed_forms.txt."""
    path = os.path.join(ROOT, "tests", "golden", "closed_forms.txt")
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == name:
                return float(parts[1])
    raise KeyError(name)


@pytest.fixture(scope="session")
def orc():
    from oracle import Oracle
    return Oracle("f32")


@pytest.fixture(scope="session")
def orc64():
    from oracle import Oracle
    return Oracle("f64")
