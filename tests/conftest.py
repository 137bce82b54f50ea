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


_reserved = False


@pytest.fixture(autouse=True)
def _gpu_workspace(request):
    """Before the first GPU test: reserve library workspace for torch's
    default stream (the library's gemm never allocates; split-K plans keep
    their partials in a workspace reserved beforehand, and the forced splits
    of these tests need up to a few hundred MiB)."""
    global _reserved
    if not _reserved and request.node.get_closest_marker("gpu") is not None:
        import dense_tiled_matrix_amd as dtm

        dtm.reserve_workspace(1 << 30)
        _reserved = True
    yield
