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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: longer CPU test")


def pytest_sessionstart(session):
    """On a machine without a GPU, build the HIP libraries (hipcc
    cross-compiles gfx950) if they do not exist yet, so that the CPU suite
    runs from a fresh checkout.  Where a GPU is visible nothing is built
    here: the libraries are built beforehand, and a missing one makes the
    tests that load it fail."""
    from pipelined_tiled_dense_amd import build as pkg_build
    missing = [lib for lib in pkg_build.LIBRARIES if not os.path.exists(os.path.join(pkg_build.HERE, lib))]
    if not missing:
        return
    import torch
    if torch.cuda.device_count() == 0:
        pkg_build.build()


@pytest.fixture(scope="session")
def oracle():
    import oracle as oracle_pkg
    return oracle_pkg.load()
