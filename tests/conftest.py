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


def pytest_collection_finish(session):
    """Compile the host programs the selected CPU tests run (decomposition checker,
    oracle mutants, sanitizer builds) now, before any test -- and so before any GPU
    test -- has run."""
    from tests import native_builds

    native_builds.prepare({item.module.__name__ for item in session.items if hasattr(item, "module")})


def pytest_sessionfinish(session, exitstatus):
    from tests import native_builds

    native_builds.cleanup()
