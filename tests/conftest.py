import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; on such a machine a missing or
    # broken library fails them loudly instead of skipping.
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def force(monkeypatch):
    """force(**names) -> rfp4_force: the binding's GEMV and GEMM calls take these kernel /
    plan overrides (gemm_rfp4_block_amd.make_force) for the rest of the test."""
    import gemm_rfp4_block_amd as R
    from tests.abi_calls import patch_binding

    def apply(**kw):
        f = R.make_force(**kw)
        patch_binding(monkeypatch, f)
        return f

    return apply
