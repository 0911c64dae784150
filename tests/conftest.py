import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The oracle mutation test runs the oracle's pins against planted mistakes:
# this names the directory holding the mutated `oracle` package to import.
_ORACLE_UNDER_TEST = os.environ.get("MLA_ORACLE_UNDER_TEST")
if _ORACLE_UNDER_TEST:
    sys.path.insert(0, _ORACLE_UNDER_TEST)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload")


@pytest.fixture
def golden_dir():
    return GOLDEN
