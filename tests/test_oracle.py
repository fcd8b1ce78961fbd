"""The fp64 oracle against its pins (CPU only).

Pins: hand-written visibility tables and hand-derived worked examples
(tests/golden/), a pure-Python dense-mask brute force, torch's CPU
scaled_dot_product_attention in float64, the invariants the method fixes and
closed forms.  See tests/oracle_pins.py for each check.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins as pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle.block_attn_f64)


def test_vs_sdpa_c1_full():
    pins.check_vs_sdpa(oracle.block_attn_f64, workloads.make("c1_tiny_d128"))


@pytest.mark.parametrize("name,cap,B", [
    ("c2_paged_d256", 200, 3),
    ("c3_global_d512", 150, 2),
    ("c4_causal_window_d256", 300, 2),
    ("c5_mixed_d512", 120, 12),
])
def test_vs_sdpa_reduced(name, cap, B):
    wl = workloads.make(name, ctx_cap=cap, B=B)
    pins.check_vs_sdpa(oracle.block_attn_f64, wl)


def test_c4_window_reduced_keeps_window_smaller_than_context():
    # a reduced C4 with W=1024 would not exercise the window; use the C4 shape
    # with a window that cuts into the context instead
    wl = workloads.make("c4_causal_window_d256", ctx_cap=200, B=2)
    wl.window = 37
    pins.check_vs_sdpa(oracle.block_attn_f64, wl)


def test_thread_count_does_not_change_results():
    wl = workloads.make("c2_paged_d256", ctx_cap=300, B=4)
    a = oracle.run_workload(wl, threads=1)
    b = oracle.run_workload(wl, threads=7)
    assert np.array_equal(a, b)


def test_row_subset_matches_full():
    wl = workloads.make("c5_mixed_d512", ctx_cap=100, B=6)
    full = oracle.run_workload(wl)
    rng = np.random.default_rng(0)
    rows = rng.choice(wl.total_q * wl.Hq, size=40, replace=False)
    sub = oracle.run_workload(wl, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, wl.D)[rows])


def test_rejects_bad_arguments():
    q = np.zeros((1, 3, 8), np.uint16)
    k = np.zeros((1, 2, 8), np.uint16)
    with pytest.raises(RuntimeError):
        oracle.block_attn_f64(q, k, k, [0], [1], [0], 3, 2, 8, 0, 1.0)   # Hq % Hkv != 0
