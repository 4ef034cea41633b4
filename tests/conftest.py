import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The oracle is compiled by __graft_entry__.build(); build it only when
    nothing is built yet (g++ takes about a second)."""
    import oracle
    if not os.path.exists(oracle.LIB):
        oracle.build()
    yield
