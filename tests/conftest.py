import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


def read_golden(name):
    """Whitespace table with '#' comments and a header row -> list of dicts."""
    path = os.path.join(ROOT, "tests", "golden", name)
    rows, header = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if header is None:
                header = parts
                continue
            rows.append({h: (p if not _isnum(p) else float(p)) for h, p in zip(header, parts)})
    return rows


def _isnum(s):
    try:
        float(s)
        return True
    except ValueError:
        return False
