import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


_INPUT_CACHE = {}


@pytest.fixture(scope="session")
def workload_inputs():
    """Cached canonical inputs per workload name: (w, q, k, v, classes) on the CPU."""
    import synth

    def get(name, **kw):
        key = (name, tuple(sorted(kw.items())))
        if key not in _INPUT_CACHE:
            w = synth.get_workload(name)
            dtype = kw.get("dtype", "bf16")
            q, k, v, cls = synth.gen_qkv(w, dtype=dtype)
            _INPUT_CACHE[key] = (w, q, k, v, cls)
        return _INPUT_CACHE[key]

    return get
