import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _host_builds():
    """Build the CPU oracle and the host generator once if they are missing."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not os.path.exists(synth.HOST_LIB):
        synth.build()
    yield
