import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def ensure_library():
    """Build libtl.so from source if it is missing or older than its sources
    (its stamp differs from the hash of the sources on disk), then import the
    binding."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_tl_build", os.path.join(ROOT, "looped_weight_shared_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.ensure_current()
    import looped_weight_shared_amd
    return looped_weight_shared_amd


def rel_rows(a, b):
    """max over rows of max|a - b| / max|b| (b is the reference)."""
    import numpy as np
    a = np.atleast_2d(np.asarray(a, dtype=np.float64))
    b = np.atleast_2d(np.asarray(b, dtype=np.float64))
    return float((np.abs(a - b).max(axis=-1) / np.abs(b).max(axis=-1)).max())


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="needs a GPU")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
