"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The work split that the planner and every kernel share (decomp.h), driven by
  tests/host/decomp_check.cpp over the five configurations' shapes and random
  edge cases: no out-of-bounds access, no signed overflow, no undefined shift.
* The fp64 oracle (oracle/oracle_f64.c), driven by tests/host/oracle_driver.c on
  exactly-sized buffers, with and without spans and row lists.
Both programs were built at session start (tests/native_builds.py) with
-fsanitize=address,undefined and -fno-sanitize-recover=all, so any report ends
the program with a non-zero status.
"""
import subprocess

import numpy as np

import workloads
from tests import native_builds


def _run(exe, stdin=""):
    r = subprocess.run([exe], input=stdin, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def _case(L, n, Hkv, G, window, rmax, tk, P, ov):
    return f"{len(L)} {Hkv} {G} {window} {rmax} {tk} {P} {ov}\n" + "\n".join(f"{a} {b}" for a, b in zip(L, n)) + "\n"


def test_decomp_under_sanitizers():
    exe = native_builds.get("decomp_check_asan")
    for name in workloads.CONFIG_ORDER:
        cfg = workloads.CONFIGS[name]
        rng = np.random.Generator(np.random.PCG64(workloads.default_seed(name)))
        L = workloads._draw_ctx(rng, cfg.ctx_law, cfg.B)
        ks = np.asarray(cfg.spec_k)
        k = ks[rng.integers(0, len(ks), size=cfg.B)] if len(ks) > 1 else np.full(cfg.B, ks[0])
        for P, ov in ((1, 0), (256, 3), (1000, 2)):
            _run(exe, _case(L, 1 + k, cfg.Hkv, cfg.Hq // cfg.Hkv, cfg.window, 80, 32, P, ov))
    rng = np.random.default_rng(17)
    for _ in range(60):
        B = int(rng.integers(1, 12))
        _run(exe, _case(rng.integers(0, 200, size=B), rng.integers(0, 30, size=B), int(rng.integers(1, 4)),
                        int(rng.integers(1, 9)), int(rng.choice([0, 1, 7, 64])), int(rng.choice([16, 48, 80])),
                        int(rng.choice([16, 32])), int(rng.integers(1, 50)), int(rng.choice([0, 1, 3]))))


def test_oracle_under_sanitizers():
    out = _run(native_builds.get("oracle_driver_asan"))
    assert int(out.split()[1]) == 60
