import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")
    config.addinivalue_line("markers", "cpu: runs without a GPU")


class _Tune:
    """Route and launch-shape overrides of libmhc (mhc_tuning_set), with the
    monkeypatch-like spelling the tests use; every override is undone when
    the test ends."""

    def __init__(self, mhc):
        self._mhc = mhc

    def setenv(self, name, value):
        self._mhc.mhc_tuning_set(name, int(value))

    def delenv(self, name, raising=False):
        self._mhc.mhc_tuning_set(name, -1)


import pytest  # noqa: E402


@pytest.fixture
def tune():
    import manifold_constrained_hyper_amd as mhc
    mhc.load()
    mhc.mhc_tuning_reset()
    yield _Tune(mhc)
    mhc.mhc_tuning_reset()
