"""The work split shared by the planner, the attention kernels and the combine
(non_causal_block_amd/csrc/decomp.h), checked on the host with g++."""
import subprocess

import numpy as np
import pytest

import workloads
from tests import native_builds


@pytest.fixture(scope="module")
def checker():
    # compiled at session start (tests/native_builds.py), never from a test body
    return native_builds.get("decomp_check")


def run(exe, L, n, Hkv, G, window, rmax, tk, P, ov=0):
    text = f"{len(L)} {Hkv} {G} {window} {rmax} {tk} {P} {ov}\n" + "\n".join(f"{a} {b}" for a, b in zip(L, n)) + "\n"
    r = subprocess.run([exe], input=text, capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    return [int(x) for x in r.stdout.split()[1:]]


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
@pytest.mark.parametrize("P", [1, 7, 256, 512, 1000])
def test_config_shapes(checker, name, P):
    cfg = workloads.CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(workloads.default_seed(name)))
    L = workloads._draw_ctx(rng, cfg.ctx_law, cfg.B)
    ks = np.asarray(cfg.spec_k)
    k = ks[rng.integers(0, len(ks), size=cfg.B)] if len(ks) > 1 else np.full(cfg.B, ks[0])
    G = cfg.Hq // cfg.Hkv
    for rmax, tk in ((80, 32), (64, 32), (16, 16)):
        for ov in (0, 2, 3, 4):
            run(checker, L, 1 + k, cfg.Hkv, G, cfg.window, rmax, tk, P, ov)


def test_random_edge_cases(checker):
    rng = np.random.default_rng(7)
    for _ in range(300):
        B = int(rng.integers(1, 20))
        L = rng.integers(0, 300, size=B)
        n = rng.integers(0, 40, size=B)
        L[rng.random(B) < 0.2] = 0
        Hkv = int(rng.integers(1, 4))
        G = int(rng.integers(1, 9))
        window = int(rng.choice([0, -3, 1, 5, 33, 1000]))
        rmax = int(rng.choice([16, 32, 48, 64, 80]))
        tk = int(rng.choice([16, 32]))
        P = int(rng.integers(1, 60))
        ov = int(rng.choice([0, 0, 1, 2, 3, 4, 7]))
        run(checker, L, n, Hkv, G, window, rmax, tk, P, ov)


def test_all_empty_requests(checker):
    assert run(checker, [5, 0, 9], [0, 0, 0], 2, 4, 0, 64, 32, 8) == [0, 0, 0]
