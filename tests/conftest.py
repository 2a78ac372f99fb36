import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def weights_dir(tmp_path_factory):
    d = os.environ.get("NVIUM_WEIGHTS_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        return d
    return str(tmp_path_factory.mktemp("weights"))


@pytest.fixture(scope="session")
def tiny_path(weights_dir):
    from synth import TINY, cached_weights
    return cached_weights(TINY, weights_dir)
