import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# The mutation test runs pin files against a copy of the oracle package with
# one planted mistake; ORACLE_DIR names the directory holding that copy.
if os.environ.get("ORACLE_DIR"):
    sys.path.insert(0, os.environ["ORACLE_DIR"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.lib()
    return oracle
