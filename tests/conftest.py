import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


_REPORTER = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_sessionstart(session):
    pm = session.config.pluginmanager
    _REPORTER.append((pm.getplugin("terminalreporter"), pm.getplugin("capturemanager")))


def progress_line(text):
    """Writes a line to the terminal even while pytest captures the test's
    output (capture suspended for the write), so that a long test shows its
    steps as they finish; returns False outside a pytest run."""
    if not _REPORTER or _REPORTER[0][0] is None:
        return False
    rep, capman = _REPORTER[0]
    if capman is not None:
        with capman.global_and_fixture_disabled():
            rep.write_line(text, flush=True)
    else:
        rep.write_line(text, flush=True)
    return True


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
