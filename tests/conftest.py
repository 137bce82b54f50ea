import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a golden fixture: '#' lines are comments, a line with a single
    word starts a section, other lines are whitespace-separated tokens."""
    sections, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            toks = line.split()
            if len(toks) == 1 and not _isnum(toks[0]):
                cur = toks[0]
                sections[cur] = []
            elif cur is None:
                sections.setdefault("_", []).append(toks)
            else:
                sections[cur].append(toks)
    return sections


def _isnum(s):
    try:
        float(s)
        return True
    except ValueError:
        return False


@pytest.fixture(scope="session")
def golden():
    return read_golden
