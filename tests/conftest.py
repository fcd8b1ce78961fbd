import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    """Compile the oracle (if its library is missing or stale) before any test touches
    the GPU: a compiler started from a process that has initialised the GPU is a
    program replacing itself in a GPU process, which must not happen."""
    import oracle

    oracle.build()
