import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def parse_golden(path):
    """Parse 'case:'-separated key/value blocks of a golden text file."""
    cases, cur = [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "case":
                cur = {"case": val}
                cases.append(cur)
            else:
                cur[key] = val
    return cases


def ints(s):
    return [int(v) for v in s.replace("|", " ").split()]


def rows_of(s, conv=int):
    return [[conv(v) for v in part.split()] for part in s.split("|")]
