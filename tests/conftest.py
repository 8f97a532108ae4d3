import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--decode-kernel", default=None, choices=("rows16", "ws", "fw"),
                     help="GPU tests: force every BF16 decode plan onto one kernel organisation "
                          "(mla_set_plan_override)")


@pytest.fixture(autouse=True)
def _plan_override(request):
    """Applies --decode-kernel to GPU tests, and restores the default plan
    choice after any test that changed it."""
    kernel = request.config.getoption("--decode-kernel")
    touched = kernel is not None or "plan_override" in request.fixturenames
    if touched:
        import mla_paged_kv_02_amd as mla
        mla.set_plan_override(kernel=kernel)
    yield
    if touched:
        import mla_paged_kv_02_amd as mla
        mla.set_plan_override()


@pytest.fixture
def plan_override(request):
    """Setter for mla_set_plan_override inside a test; the kernel defaults
    to --decode-kernel's."""
    import mla_paged_kv_02_amd as mla
    default_kernel = request.config.getoption("--decode-kernel")

    def set_(merge=None, kernel=None):
        mla.set_plan_override(kernel=kernel or default_kernel, merge=merge)
    return set_


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; skip them loudly rather than
    # letting them fall back to anything else.
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
