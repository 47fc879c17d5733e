import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def cuda():
    """The torch device for GPU tests; fails (not skips) when a gpu-marked test
    runs without a GPU, so that a silent skip cannot pass for a green run."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Repeat the parity lines the GPU tests reported (whole-output error
    ratios and exact comparisons), so they stay visible under -q."""
    mod = sys.modules.get("tests.gpu_util")
    lines = getattr(mod, "SUMMARY", None) if mod is not None else None
    if lines:
        terminalreporter.write_sep("-", "parity summary")
        for line in lines:
            terminalreporter.write_line(line)
