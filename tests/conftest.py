import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # The binding fails loudly without libmtla.so; build it here only if nothing
    # is built yet (a cross-compile for gfx950 that needs no GPU).
    from tests.libmtla import ensure_built
    ensure_built()
