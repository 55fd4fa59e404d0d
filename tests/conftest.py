import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    from oracle import DEFAULT_LIB, Oracle
    from oracle.build import SRC, build
    if not os.path.exists(DEFAULT_LIB) or os.path.getmtime(DEFAULT_LIB) < os.path.getmtime(SRC):
        build()
    return Oracle()
