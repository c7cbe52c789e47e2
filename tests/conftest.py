import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU-only statistical test")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    parity = sys.modules.get("tests.parity")
    ties = getattr(parity, "NEAR_TIES", None)
    if ties is None:
        return
    terminalreporter.write_line(
        f"near-ties (GPU != oracle with the oracle's deciding margin < 1e-6 relative): {len(ties)}")
    for label, b, m in ties[:50]:
        terminalreporter.write_line(f"  {label} request {b}: margin {m:.3e}")
