import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def root():
    return ROOT


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def poison_workspaces(monkeypatch):
    """Every workspace the binding allocates or is handed is filled with 0xFF
    bytes before the call (its contents are undefined by contract), so a
    kernel that reads workspace memory it has not written in the same call
    (a stale table, a split-K partial) sees NaN or -1 instead of leftovers
    that happen to be right."""
    from mixture_experts_layer_exclusive_amd import api

    real = api._workspace

    def poisoned(p, op, device, ws):
        ws, nbytes = real(p, op, device, ws)
        ws.view(-1).view(api.torch.uint8).fill_(0xFF)
        return ws, nbytes

    monkeypatch.setattr(api, "_workspace", poisoned)
