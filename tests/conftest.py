"""Shared test setup.

Markers: `gpu` tests need an MI355X (gfx950) and libmxstore.so; everything
else runs on the CPU.  Both the HIP library and the C oracle are built on
first use when absent (the driver's build step normally did it already).
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and libmxstore.so")


@pytest.fixture(scope="session")
def mxlib():
    """The HIP library, built if missing (never a fallback)."""
    from mxfp4_paged_cache_store_amd import _abi, build

    if not os.path.exists(build.LIB_PATH):
        build.build()
    return _abi.lib()


@pytest.fixture(scope="session")
def device(mxlib):
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu test on a machine without a GPU: run with -m 'not gpu' here")
    return torch.device("cuda:0")
