import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: long CPU test")


def to_np(t):
    """torch tensor -> numpy; bf16 becomes its uint16 bit pattern."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
