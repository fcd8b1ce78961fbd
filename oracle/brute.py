"""Pure-Python brute force of DFlash block attention, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

A second formulation of the same definition as ``oracle_f64.c``, written
independently: instead of a [lo, hi] key range it materialises, for every
query, the dense boolean visibility row over all T = L + n keys of its
request straight from the rules on the pages, and it uses exactly rounded
sums (``math.fsum``) in place of running sums.

Visibility (kenforever1, "DFlash + Gemma 4 31B-it" notes, section "why
non-causal attention is needed"; vLLM PR #43445 report, "key code"):
  * a non-causal block is processed as a whole: every key of the request;
  * a causal query sees only itself and the keys to its left;
  * a sliding window of W keys keeps only the W keys that end at the query's
    own position (W <= 0: no window).
"""
from __future__ import annotations

import math

import numpy as np


def visible(L: int, n: int, is_causal: bool, window: int, i: int, j: int, spans=()) -> bool:
    """Whether query i of a block (context L, block n) may attend to key j.

    ``spans``: the request's bidirectional spans, (start, end) key-position
    pairs: two positions inside one span see each other in both directions,
    even in a causal request (the mm-prefix case)."""
    T = L + n
    pos = L + i                      # the query's own key position
    if not (0 <= j < T):
        return False
    together = any(s <= pos < e and s <= j < e for s, e in spans)
    if is_causal and j > pos and not together:   # nothing to the right, except inside a span
        return False
    if window > 0 and pos - j >= window:   # only the W keys ending at pos
        return False
    return True


def mask_matrix(L: int, n: int, is_causal: bool, window: int, spans=()) -> np.ndarray:
    return np.array([[visible(L, n, is_causal, window, i, j, spans) for j in range(L + n)] for i in range(n)],
                    dtype=bool)


def block_attn(q, k, v, ctx_lens, block_lens, causal, Hq, Hkv, D, window, scale, spans=None):
    """q [total_q, Hq, D], k/v [total_kv, Hkv, D] as float64 arrays (bf16 values).

    Returns float64 [total_q, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    G = Hq // Hkv
    out = np.zeros((q.shape[0], Hq, D), dtype=np.float64)
    qs = 0
    ks = 0
    for r in range(len(ctx_lens)):
        L, n = int(ctx_lens[r]), int(block_lens[r])
        c = bool(causal[r]) if causal is not None else False
        T = L + n
        M = mask_matrix(L, n, c, window, () if spans is None else spans[r])
        for i in range(n):
            for h in range(Hq):
                g = h // G
                qrow = [float(x) for x in q[qs + i, h]]
                logits = []
                for j in range(T):
                    if M[i, j]:
                        krow = k[ks + j, g]
                        logits.append(scale * math.fsum(qrow[d] * float(krow[d]) for d in range(D)))
                    else:
                        logits.append(None)
                mx = max(x for x in logits if x is not None)
                w = [math.exp(x - mx) if x is not None else 0.0 for x in logits]
                s = math.fsum(w)
                for d in range(D):
                    out[qs + i, h, d] = math.fsum(w[j] * float(v[ks + j, g, d]) for j in range(T)) / s
        qs += n
        ks += T
    return out
