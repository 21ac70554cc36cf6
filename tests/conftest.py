import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and binding; GPU tests fail loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import rl_post_loss_amd as rpl
    rpl.load_library()  # raises if the shared library was not built
    return rpl


def pytest_sessionstart(session):
    # GRPO_TEST_LIB: run the tests against another build of libgrpo (the
    # host-sanitized build of tests/test_host_sanitizers.py); unset on every
    # ordinary run
    path = os.environ.get("GRPO_TEST_LIB")
    if path:
        from rl_post_loss_amd import _abi
        _abi._lib = _abi.load_library(path)
