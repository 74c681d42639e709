import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


class _Tuning:
    """Sets the library's tuning environment variables for one test: each
    change goes through monkeypatch, then the library reads them again (it
    reads them once, at its first call)."""

    def __init__(self, mp):
        self.mp = mp

    @staticmethod
    def reload():
        import softmax_cross_entropy_fwd_amd as ce
        ce.reload_tuning()

    def setenv(self, name, value):
        self.mp.setenv(name, value)
        self.reload()

    def delenv(self, name, raising=True):
        self.mp.delenv(name, raising=raising)
        self.reload()


@pytest.fixture
def tuning(monkeypatch):
    t = _Tuning(monkeypatch)
    yield t
    monkeypatch.undo()
    t.reload()
