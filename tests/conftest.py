import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # the tests run what is built; they build only when nothing is
    import __graft_entry__
    __graft_entry__.build_if_missing()


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
