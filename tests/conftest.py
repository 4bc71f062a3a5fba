import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU in this environment")
    import torch
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    h = sys.modules.get("engram_harness") or sys.modules.get("tests.engram_harness")
    st = getattr(h, "f32_stats", None)
    if not st or not st["checks"]:
        return
    terminalreporter.write_line(
        "fp32 parity over %d checks: elementwise relative error on %d elements with |ref| >= row RMS: "
        "max %.2e (bound 1e-5); the other %d elements: max |d| / row RMS %.2e (floor 1e-5)"
        % (st["checks"], st["n_large"], st["max_rel_large"], st["n_small"], st["max_abs_over_rms_small"]))
