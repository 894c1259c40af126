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
    """The HIP binding, loaded from the in-tree library; a GPU test fails if it is absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a visible GPU")
    import gated_linear_recurrence_amd as glr
    glr.load_library()
    return glr


@pytest.fixture(autouse=True)
def _no_workspace_errors(request):
    """After every GPU test: no scan call may have left an error bit in any live workspace.

    The error word is sticky, so a bounded wait that ran out anywhere in the
    test (a look-back across workgroups or a wait between the waves of one)
    fails the test that caused it.
    """
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import gated_linear_recurrence_amd as glr
    glr.check_errors()
