import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run (flushed) so that a run cut short
    # still names it.
    for item in items:
        if item.get_closest_marker("gpu") is not None:
            item.add_marker(pytest.mark.usefixtures("_announce_gpu_case"))


@pytest.fixture
def _announce_gpu_case(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield


class _Tune:
    """Launch-shape tuning overrides for one test (q_tuning_set through the
    binding); every key the test set is cleared when it ends."""

    def __init__(self):
        self.keys = set()

    def set(self, name, value):
        from dequant_gemv_rtn_amd import binding

        binding.set_tuning(name, int(value))
        self.keys.add(name)

    def clear(self, name):
        from dequant_gemv_rtn_amd import binding

        binding.clear_tuning(name)


@pytest.fixture
def tune():
    t = _Tune()
    yield t
    if t.keys:
        from dequant_gemv_rtn_amd import binding

        for name in t.keys:
            binding.clear_tuning(name)
