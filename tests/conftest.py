import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def dsa():
    """The HIP library binding; GPU tests fail loudly if it cannot be loaded."""
    if not gpu_available():
        pytest.skip("no GPU")
    import sparse_attention_05_amd as dsa_mod
    dsa_mod.load()
    return dsa_mod


def pytest_terminal_summary(terminalreporter):
    """Per-config parity statistics gathered by the GPU parity tests (near-tie swaps,
    planted-token recall, worst errors)."""
    try:
        import parity
    except ImportError:
        return
    if not parity.REPORT:
        return
    import json
    terminalreporter.section("parity statistics per config")
    for name in sorted(parity.REPORT):
        terminalreporter.write_line("%s: %s" % (name, json.dumps(parity.REPORT[name], sort_keys=True)))
    path = os.environ.get("DSA_PARITY_REPORT")
    if path:
        with open(path, "w") as fh:
            json.dump(parity.REPORT, fh, indent=1, sort_keys=True)
