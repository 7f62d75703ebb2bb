"""Shared pytest configuration: the `gpu` marker, the repository root on sys.path, and one
device initialisation per session before any GPU test builds its inputs.

The seeded input generators fill CPU tensors on a thread pool.  A process whose first device
touch came after that thread-pool work ended in a host segmentation fault inside torch's first
device initialisation, while every process that touched the device first ran cleanly.  So a
session that runs GPU tests initialises the device (and allocates once on it) before the first
test, whatever order the test files run in.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library through its C ABI")


@pytest.fixture(scope="session", autouse=True)
def _device_first(request):
    """Initialise the GPU once, before any test generates inputs, when GPU tests were selected."""
    if any(item.get_closest_marker("gpu") for item in request.session.items):
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
            torch.zeros(1, device="cuda:0").add_(1)
            torch.cuda.synchronize()
    yield
