import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large-size parity case")


def read_golden_table(name):
    """Rows of 'index value' from a golden text file (comment lines start with #)."""
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            i, v = line.split()
            vals[int(i)] = v
    return [vals[i] for i in range(len(vals))]


@pytest.fixture(scope="session")
def nf4_literals_8dp():
    return read_golden_table("nf4_table_8dp.txt")


@pytest.fixture(scope="session")
def nf4_literals_4dp():
    return read_golden_table("nf4_table_4dp.txt")
