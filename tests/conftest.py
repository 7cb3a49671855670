import os
import sys

import pytest

# Every forward the tests make through the Python binding clears and then
# checks its workspace's error word (a hand-off wait that gave up fails the test).
os.environ.setdefault("LA_CHECK_WAITS", "1")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU-only cases")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()
