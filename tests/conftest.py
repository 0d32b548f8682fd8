import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size layer; minutes on the CPU")


@pytest.fixture(scope="session")
def orc():
    from oracle.oracle import Oracle, LIBRARY, SOURCE, compile_library
    if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_library()
    return Oracle(LIBRARY)
