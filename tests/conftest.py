import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library, built first if nothing is built yet."""
    from cross_cu_load_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.load()


@pytest.fixture(scope="session")
def dev(lib):
    """(compute units, XCDs) of cuda:0; skips when no GPU is visible."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(0)
    from cross_cu_load_amd import binding
    return binding.device_query(0)


def pytest_sessionfinish(session, exitstatus):
    """Writes the parity margins the GPU tests collected to $CC_PARITY_LOG (if set)."""
    path = os.environ.get("CC_PARITY_LOG")
    if not path:
        return
    try:
        import gpu_helpers
    except ImportError:
        return
    if gpu_helpers.MARGINS:
        import json
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(gpu_helpers.MARGINS, f, indent=1)
