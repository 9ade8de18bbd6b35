import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


MODEL_DIR = os.environ.get("PPX_MODEL_DIR", "/tmp/ppx_models")


@pytest.fixture(scope="session")
def model_dir():
    os.makedirs(MODEL_DIR, exist_ok=True)
    return MODEL_DIR
