import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture
def tune():
    """Setter for the library's test hooks (include/qw_tuning.h); every hook
    set through it returns to the automatic choice after the test."""
    from bit_weight_quantized_qw_amd import qw
    keys = []

    def set_(key, value):
        qw.qw_tune_set(key, value)
        keys.append(key)

    yield set_
    for k in keys:
        qw.qw_tune_set(k, qw.QW_TUNE_AUTO)
