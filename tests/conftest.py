import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle work")


@pytest.fixture(scope="session")
def gpu():
    """The GPU device; GPU tests refuse to run on a silent fallback."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import trellis_quantized_linear_tf_amd as tq

    tq.load()  # raises if the HIP library is missing
    name = torch.cuda.get_device_properties(0).gcnArchName
    print(f"[gpu] device 0: {name}", flush=True)
    return torch.device("cuda:0")
