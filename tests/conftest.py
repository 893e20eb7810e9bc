import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# The oracle's mutation check runs the pins against planted-mistake copies of
# the oracle package: this variable names the folder that holds such a copy.
_ORACLE_COPY = os.environ.get("SA_ORACLE_COPY_DIR")
if _ORACLE_COPY:
    sys.path.insert(0, _ORACLE_COPY)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads")
