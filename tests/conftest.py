import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (runs the HIP kernels through the C ABI)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Kink bookkeeping of the BatchNorm parity cases: how many elements
    were moved off an activation kink, or decided by the GPU's own side on
    unedited inputs."""
    try:
        from tests._parity import KINK_LOG
    except Exception:
        return
    if KINK_LOG:
        terminalreporter.write_sep("-", "activation kinks in the parity inputs")
        for line in KINK_LOG:
            terminalreporter.write_line(line)
