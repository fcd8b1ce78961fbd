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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The full-size parity table of this session (GPU runs only)."""
    helpers = sys.modules.get("tests.gpu_helpers")
    rows = getattr(helpers, "PARITY_REPORT", None)
    if not rows:
        return
    tr = terminalreporter
    tr.write_line("")
    tr.write_line("full-size parity against the fp64 oracle (every output element):")
    tr.write_line("| workload | kernel | rows | max abs err | mean abs err | rel RMS err | oracle s |")
    tr.write_line("|---|---|---|---|---|---|---|")
    for r in rows:
        tr.write_line(f"| {r['workload']} | {r['kernel']} | {r['rows']} | {r['max_abs']:.2e} | {r['mean_abs']:.2e} | "
                      f"{r['rel_rms']:.2e} | {r['oracle_s']:.2f} |")
    path = os.environ.get("DFLASH_PARITY_REPORT")
    if path:
        import json

        with open(path, "w") as f:
            json.dump(rows, f, indent=1)
