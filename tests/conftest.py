import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of host time)")


@pytest.fixture
def progress(request):
    """A print that reaches the terminal at once, past pytest's output capture.
    Long tests report each step they finish (an oracle task done, a member
    checked), so that minutes of host-side oracle work never look like a hung
    run to a caller that watches the output."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def say(msg, **_):
        if capman is None:
            print(msg, flush=True)
            return
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)

    return say
