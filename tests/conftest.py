import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded through the Python binding; skips when no GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kronecker_factored_gptq_amd as bk
    bk.lib()  # raises if the extension is missing
    return bk


@pytest.fixture
def progress(request):
    """say(msg): a progress line on the terminal while output is captured,
    for tests whose oracle work runs for minutes without a result line."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def say(msg):
        if capman is None:
            print(f"[progress] {msg}", flush=True)
            return
        with capman.global_and_fixture_disabled():
            print(f"[progress] {msg}", flush=True)
    return say
