import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _number(text):
    """An integer where the text is one, else a float (decimal fixtures)."""
    try:
        return int(text)
    except ValueError:
        return float(text)


def load_golden(name):
    """Parse a fixture: blocks of `LABEL rows cols` followed by rows of numbers."""
    blocks = {}
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
    i = 0
    while i < len(lines):
        label, r, c = lines[i].split()
        r, c = int(r), int(c)
        rows = [[_number(x) for x in lines[i + 1 + t].split()] for t in range(r)]
        assert all(len(row) == c for row in rows), (name, label)
        blocks[label] = rows
        i += 1 + r
    return blocks


def load_grid_counts():
    out = []
    with open(os.path.join(GOLDEN, "grid_counts.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                out.append([int(x) for x in ln.split()])
    return out


@pytest.fixture(scope="session", autouse=True)
def _hip_library_built():
    """Build the HIP library once if nothing is built yet (no rebuild otherwise)."""
    from dense_gemm_07_amd.build import LIB, build
    if not os.path.exists(LIB):
        build()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle
