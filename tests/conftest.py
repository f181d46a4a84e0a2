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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()


@pytest.fixture(scope="session", autouse=True)
def _hip_library_current():
    """Rebuild libmambascan.so before any test if its sources changed since it was built."""
    from selective_state_space_72_amd import build as hip_build
    hip_build.ensure_built(verbose=False)
