"""KV page size on the HIP path: the same logical K/V, paged with page sizes
from 1 to 256 keys, must give bitwise-identical outputs.

The work split, the tiles and every summation order are independent of the
page size; only the key addresses change.  Pages of at least 16 keys and
smaller pages are located by different kernel instances (two page ids per
32-key tile versus one per key), and keys past a request's end read its last
key, which sits in a different place for every page size.  Page tails are
NaN-poisoned, so any read of a slot outside the request shows up as a
non-finite output.  The page-16 result is also checked against the fp64
oracle at the usual bar.
"""
import dataclasses

import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import oracle
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

PAGE_SIZES = [1, 2, 4, 8, 16, 32, 64, 256]

CASES = [
    # (Hq, Hkv, D, ctx_lens, block_lens, causal, window)
    (32, 4, 512, [1000, 37, 0, 517], [9, 9, 5, 16], [0, 1, 1, 0], 0),    # 72 rows; 128 rows in two groups
    (32, 4, 512, [1000, 37, 0, 517], [9, 9, 5, 16], [1, 1, 0, 1], 100),  # windowed
    (16, 4, 256, [300, 15, 16, 1200], [9, 1, 16, 9], [1, 0, 1, 0], 0),
    (8, 2, 128, [31, 32, 33, 700], [16, 9, 1, 9], [0, 1, 0, 1], 40),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def repage(wl: workloads.Workload, page_size: int, seed: int) -> workloads.Workload:
    """The same logical K/V in pages of `page_size` keys (seeded permutation, poisoned tails)."""
    kv_lens = wl.ctx_lens.astype(np.int64) + wl.block_lens.astype(np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    table, num_pages = workloads.page_layout(kv_lens, page_size, rng, extra_pages=2)
    return dataclasses.replace(
        wl, page_size=page_size, page_table=table,
        k_pages=workloads.scatter_to_pages(wl.k, kv_lens, table, num_pages, page_size, True),
        v_pages=workloads.scatter_to_pages(wl.v, kv_lens, table, num_pages, page_size, True))


def bits(o: torch.Tensor) -> torch.Tensor:
    return o.cpu().view(torch.int16)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_page_size_invariance_bitwise(case):
    Hq, Hkv, D, L, n, c, W = CASES[case]
    wl = workloads.build(len(L), Hq, Hkv, D, L, n, c, window=W, seed=700 + case, page_size=16, extra_pages=2)
    ref = oracle.run_workload(wl)
    for nwg in (0, 7):
        base = H.run(wl, kernel=nb.DFLASH_KERNEL_MFMA, num_workgroups=nwg)
        H.assert_parity(H.to_f64(base), ref, f"case {case} page 16 wg={nwg}")
        for P in PAGE_SIZES:
            if P == 16:
                continue
            got = H.run(repage(wl, P, seed=900 + P), kernel=nb.DFLASH_KERNEL_MFMA, num_workgroups=nwg)
            assert torch.equal(bits(got), bits(base)), f"case {case} page {P} wg={nwg} differs from page 16"


def test_spans_with_small_and_large_pages_bitwise():
    # bidirectional spans use their own kernel instances, again split by page size
    wl = workloads.build(3, 16, 4, 256, [300, 64, 900], [9, 16, 9], [1, 1, 1], seed=77, page_size=16,
                         extra_pages=2)
    spans = workloads.draw_spans(wl.ctx_lens, wl.block_lens, seed=5, max_prefix_span=64)
    ref = oracle.run_workload(wl, spans=spans)
    base = H.run(wl, kernel=nb.DFLASH_KERNEL_MFMA, spans=spans)
    H.assert_parity(H.to_f64(base), ref, "spans page 16")
    for P in (2, 8, 64):
        got = H.run(repage(wl, P, seed=910 + P), kernel=nb.DFLASH_KERNEL_MFMA, spans=spans)
        assert torch.equal(bits(got), bits(base)), f"spans page {P} differs from page 16"
