import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_sessionstart(session):
    # A library built from other sources than the ones in the tree would test
    # the wrong code: refuse to run against it.  (Checked on the file: the
    # library is loaded only after torch has initialised the GPU runtime.)
    from block_diffusion_speculative_amd import _lib
    if os.path.exists(_lib.LIB_PATH) and not _lib.file_is_fresh():
        raise pytest.UsageError(
            f"{_lib.LIB_PATH} was built from other sources than the ones in the tree "
            "(dflash_build_id differs from the source digest): rebuild with __graft_entry__.build()")


def pytest_collection_modifyitems(config, items):
    # GPU tests need the device; when run without one they are skipped with a reason
    # rather than silently passing.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
