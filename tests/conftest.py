import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a ``key: values`` golden file; repeated keys become lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out.setdefault(key.strip(), []).append(val.split())
    return out


@pytest.fixture
def golden():
    return read_golden


def ensure_built():
    """Build libi8mm.so only if it is not there (the GPU machine gets it prebuilt)."""
    from int8_mixed_precision_detect_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from int8_mixed_precision_detect_amd import build
        build.build()
    return _lib.LIB_PATH


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
