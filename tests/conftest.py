import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


@pytest.fixture(scope="session")
def sf_weights_f32():
    from oracle.weights import make_weights
    return make_weights("sortformer", 0)


@pytest.fixture(scope="session")
def sf_weights_full():
    from oracle.weights import make_weights
    return make_weights("sortformer", 7, full_random=True)


@pytest.fixture(scope="session")
def nm_weights_full():
    from oracle.weights import make_weights
    return make_weights("nemotron", 9, full_random=True)
