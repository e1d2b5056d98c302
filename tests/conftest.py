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
def tiny_weights():
    from seeded_inputs import generate_weights, get_config
    return generate_weights(get_config("tiny"))


@pytest.fixture(scope="session")
def tiny_model(tiny_weights):
    from oracle import Fp64Model
    return Fp64Model(tiny_weights)


@pytest.fixture(scope="session")
def q8b_device():
    """Seeded 8B-shaped weights packed on cuda:0 (shared by the 8B and 32K tests)."""
    from greedy_block_verification_amd.session import DeviceModel
    from seeded_inputs import generate_weights, get_config
    w = generate_weights(get_config("q8b"))
    return DeviceModel(w), w
