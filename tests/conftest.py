import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP device (MI355X); run with -m gpu")
    config.addinivalue_line("markers", "slow: full-size parity cases (GiB inputs)")


def _reload_library_hooks(name):
    # libblake3_gpu.so reads its BLAKE3_GPU_* test hooks once, when it is loaded: after a
    # change, ask it to read them again (every handle of the process shares one copy)
    if not name.startswith("BLAKE3_GPU_"):
        return
    import blake3_merkle_tree_amd as b3
    try:
        lib = b3._load()
    except ImportError:  # not built (or a test has hidden it): nothing to tell
        return
    lib.blake3_gpu_debug_reload_env()


class _HookAwareMonkeyPatch(pytest.MonkeyPatch):
    """pytest's MonkeyPatch, except that setting, deleting or restoring a BLAKE3_GPU_*
    environment variable also makes the library re-read its test hooks."""

    def setenv(self, name, value, prepend=None):
        super().setenv(name, value, prepend)
        _reload_library_hooks(name)

    def delenv(self, name, raising=True):
        super().delenv(name, raising)
        _reload_library_hooks(name)

    def undo(self):
        super().undo()
        _reload_library_hooks("BLAKE3_GPU_")


@pytest.fixture
def monkeypatch():
    mp = _HookAwareMonkeyPatch()
    yield mp
    mp.undo()
