import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large-scene test (minutes on the CPU)")


@pytest.fixture(scope="session")
def tiny_scene():
    import scenegen
    return scenegen.make_config(1)


@pytest.fixture(scope="session")
def small_scene():
    import scenegen
    return scenegen.make_config(2)
