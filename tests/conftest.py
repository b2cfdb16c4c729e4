import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a tests/golden fixture: 'key: v1 v2 ... [tol T]' per line, '#' comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(":", 1)
            tol = None
            if " tol " in " " + rest:
                rest, t = rest.rsplit("tol", 1)
                tol = float(t)
            out[key.strip()] = ([float(x) for x in rest.split()], tol)
    return out


@pytest.fixture
def golden():
    return load_golden
