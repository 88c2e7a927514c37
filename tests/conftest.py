import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The library is built in-tree ahead of time; build it here only if nothing is built.
    if not os.path.exists(os.path.join(ROOT, "combine_lds_atomic_amd", "libmoe_ep.so")):
        import runpy   # by path: importing the package itself needs the built library
        runpy.run_path(os.path.join(ROOT, "combine_lds_atomic_amd", "build.py"))["build"]()


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; skip them loudly rather than fail when none is present
    # and the run did not ask for them explicitly.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu or config.getoption("-m", default="").strip() == "gpu":
        return   # an explicit `-m gpu` run must fail loudly without a device
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
