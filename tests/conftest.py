import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


@pytest.fixture(scope="session")
def gdn_lib():
    """The HIP-backed binding; fails loudly when no GPU or no library is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but torch.cuda.is_available() is False")
    import hybrid_model_linear_amd as gdn
    gdn.load()          # raises when libgdn.so is missing
    return gdn
