import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


_CONFIG = None


def pytest_configure(config):
    global _CONFIG
    _CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def progress(msg):
    """A progress line on the terminal's stderr even while pytest captures
    the test's output (long GPU comparisons are then seen to advance)."""
    capman = _CONFIG.pluginmanager.getplugin("capturemanager") if _CONFIG else None
    if capman is None:
        print(msg, file=sys.stderr, flush=True)
        return
    with capman.global_and_fixture_disabled():
        print(msg, file=sys.stderr, flush=True)


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden
