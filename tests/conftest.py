"""Shared pytest set-up: the ``gpu`` marker, import path, and a build of the
native libraries when none is present yet."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    pkg = os.path.join(ROOT, "mixed_precision_dense_tiled_amd")
    need = [os.path.join(ROOT, "oracle", "liboracle.so"), os.path.join(pkg, "libmpdt.so"),
            os.path.join(pkg, "libmpdt_probes.so"), os.path.join(pkg, "libmpdt_clock.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_ok():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
