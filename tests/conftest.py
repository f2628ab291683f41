import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# A copy of oracle/ with a planted mistake (tests/test_oracle_mutants.py) is
# imported in place of oracle/ when its directory is named here.
if os.environ.get("HG_ORACLE_DIR"):
    sys.path.insert(0, os.environ["HG_ORACLE_DIR"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    from oracle import hashgrid_oracle
    return hashgrid_oracle
