"""Pins of the block K/V append oracle (oracle/append.py).

* A hand-worked case: two requests, page size 4, where every block token's
  (page, slot) is written out below from the definition.
* Round trip: pages holding only the context (block slots poisoned) plus the
  appended block rows equal the cache built from the full logical K/V by the
  input generator -- bit for bit, block slots included, every other slot
  untouched -- over several page sizes, empty blocks and empty contexts.
"""
import numpy as np
import pytest

import workloads
from oracle.append import block_kv_append


def test_hand_worked_example():
    # request 0: L=3, n=2 -> positions 3, 4; page size 4 -> (page_table[0,0], slot 3), (page_table[0,1], slot 0)
    # request 1: L=0, n=3 -> positions 0, 1, 2 -> (page_table[1,0], slots 0, 1, 2)
    P, Hkv, D = 4, 1, 2
    page_table = np.array([[5, 2], [0, 7]], dtype=np.int32)
    k_pages = np.zeros((8, P, Hkv, D), dtype=np.uint16)
    v_pages = np.zeros_like(k_pages)
    k_new = np.arange(1, 11, dtype=np.uint16).reshape(5, Hkv, D)        # rows t = 0..4
    v_new = (100 + np.arange(1, 11, dtype=np.uint16)).reshape(5, Hkv, D)
    k_out, v_out = block_kv_append(k_pages, v_pages, k_new, v_new, page_table, np.array([3, 0]), np.array([2, 3]))
    want = np.zeros_like(k_pages)
    want[5, 3, 0] = [1, 2]     # request 0, token 0 (position 3)
    want[2, 0, 0] = [3, 4]     # request 0, token 1 (position 4)
    want[0, 0, 0] = [5, 6]     # request 1, token 0
    want[0, 1, 0] = [7, 8]
    want[0, 2, 0] = [9, 10]
    assert np.array_equal(k_out, want)
    assert np.array_equal(v_out, np.where(want != 0, want + 100, 0))
    assert (k_pages == 0).all()  # inputs untouched


@pytest.mark.parametrize("page_size", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("seed", [0, 1])
def test_append_restores_the_full_cache(page_size, seed):
    rng = np.random.default_rng(seed)
    B = 5
    ctx = rng.integers(0, 70, size=B)
    blk = rng.integers(0, 17, size=B)
    ctx[0], blk[1] = 0, 0  # an empty context and an empty block
    wl = workloads.build(B, 4, 2, 16, ctx, blk, np.zeros(B, dtype=np.uint8), seed=seed, page_size=page_size,
                         extra_pages=2)
    k_new, v_new, k_ctx, v_ctx = workloads.split_block_kv(wl)
    assert k_new.shape == (wl.total_q, wl.Hkv, wl.D)
    k_out, v_out = block_kv_append(k_ctx, v_ctx, k_new, v_new, wl.page_table, wl.ctx_lens, wl.block_lens)
    assert np.array_equal(k_out, wl.k_pages) and np.array_equal(v_out, wl.v_pages)
    # the block slots really were poisoned before the append
    if wl.total_q:
        assert not np.array_equal(k_ctx, wl.k_pages)
