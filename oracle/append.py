"""Oracle for the block K/V append (test infrastructure only; see the package
docstring for who may use it).

Definition (kenforever1 "DFlash + Gemma 4 31B-it" notes, "why non-causal
attention is needed": the block's queries attend to the context K/V together
with the block's own K/V; both live in one paged cache): block token i of
request r is key position p = L + i, stored at page page_table[r, p // P],
slot p % P.  Row t of k_new / v_new is block token t - q_start[r] of the
request whose block contains t (rows packed in request order).
"""
from __future__ import annotations

import numpy as np


def block_kv_append(k_pages: np.ndarray, v_pages: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                    page_table: np.ndarray, ctx_lens: np.ndarray, block_lens: np.ndarray):
    """Return copies of k_pages / v_pages ([num_pages, P, Hkv, D]) with every block row written."""
    k_out = k_pages.copy()
    v_out = v_pages.copy()
    P = k_pages.shape[1]
    t = 0
    for r in range(len(ctx_lens)):
        L = int(ctx_lens[r])
        for i in range(int(block_lens[r])):
            p = L + i
            page = int(page_table[r, p // P])
            k_out[page, p % P] = k_new[t]
            v_out[page, p % P] = v_new[t]
            t += 1
    return k_out, v_out
