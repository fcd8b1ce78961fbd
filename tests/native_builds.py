"""Host programs the CPU tests compile, built once per session before any test runs.

conftest.py calls ``prepare`` from ``pytest_collection_finish``: every compiler is
started before the first test, so never from a process that a GPU test has
already initialised (a compiler started from a GPU-initialised process is a
program replacing itself in a GPU process).  Tests only look their programs up
here; a missing entry is an error, never a reason to compile inside a test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "non_causal_block_amd", "csrc")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle_f64.c")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

_built: dict = {}
_dir = None


def _out(name: str) -> str:
    global _dir
    if _dir is None:
        _dir = tempfile.mkdtemp(prefix="dflash_native_")
    return os.path.join(_dir, name)


def _decomp_check(sanitized: bool) -> str:
    exe = _out("decomp_check_asan" if sanitized else "decomp_check")
    cmd = ["g++", "-O1" if sanitized else "-O2", "-std=c++17", "-I", CSRC, *(SANITIZE if sanitized else []),
           os.path.join(HERE, "host", "decomp_check.cpp"), "-o", exe]
    subprocess.check_call(cmd)
    return exe


def _oracle_driver() -> str:
    exe = _out("oracle_driver_asan")
    subprocess.check_call(["gcc", "-O1", "-ffp-contract=off", "-pthread", *SANITIZE, ORACLE_C,
                           os.path.join(HERE, "host", "oracle_driver.c"), "-o", exe, "-lm"])
    return exe


def _mutants() -> dict:
    from tests.test_oracle_mutants import MUTANTS

    src = open(ORACLE_C).read()
    libs = {}
    for name, (old, new) in MUTANTS.items():
        if src.count(old) != 1:
            raise RuntimeError(f"mutation anchor for {name} not found exactly once")
        c = _out(f"mutant_{name}.c")
        with open(c, "w") as fh:
            fh.write(src.replace(old, new))
        so = _out(f"libmutant_{name}.so")
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", c, "-o", so, "-lm"])
        libs[name] = so
    return libs


BUILDERS = {
    "tests.test_decomp": lambda: {"decomp_check": _decomp_check(False)},
    "tests.test_oracle_mutants": lambda: {"mutants": _mutants()},
    "tests.test_sanitizers": lambda: {"decomp_check_asan": _decomp_check(True), "oracle_driver_asan": _oracle_driver()},
}


def prepare(modules) -> None:
    """Build what the selected test modules need (module names as imported)."""
    for mod, fn in BUILDERS.items():
        short = mod.split(".")[-1]
        if any(m == mod or m.endswith("." + short) or m == short for m in modules):
            _built.update(fn())


def get(name: str):
    if name not in _built:
        raise RuntimeError(f"{name} was not built at session start (tests/conftest.py)")
    return _built[name]


def cleanup() -> None:
    if _dir and os.path.isdir(_dir):
        shutil.rmtree(_dir, ignore_errors=True)
