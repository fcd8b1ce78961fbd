"""Oracle for DFlash2's in-block grouped dynamic depthwise convolution (test
infrastructure only; see the package docstring for who may use it).

Definition (prhub summary of vLLM PR #52816, "DFlash2: local convolution +
candidate selector", section "motivation"): for each request's block and each
position i and channel c,
    out[i,c] = sum_t (base[t,c] + delta[i,t,g(c)]) * x[i-t,c],
with taps that reach before the block's first position equal to zero.  Channel
groups are contiguous: g(c) = c // (C // G) (a reading; the page does not
spell out the grouping).  Evaluated sequentially -- position by position, tap
by tap -- in float64, as the PR's own test compares against a sequential
reference.
"""
from __future__ import annotations

import numpy as np


def block_conv_f64(x: np.ndarray, base: np.ndarray, delta: np.ndarray, block_lens, groups: int) -> np.ndarray:
    """x [total_q, C], base [taps, C], delta [total_q, taps, G] (any float dtype) -> float64 [total_q, C]."""
    x = np.asarray(x, dtype=np.float64)
    base = np.asarray(base, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    total_q, C = x.shape
    taps = base.shape[0]
    g_of_c = np.arange(C) // (C // groups)
    out = np.zeros((total_q, C), dtype=np.float64)
    start = 0
    for n in np.asarray(block_lens, dtype=np.int64):
        n = int(n)
        for i in range(n):
            row = start + i
            for t in range(taps):
                if i - t < 0:
                    break  # the tap reaches before the block: zero
                coef = base[t] + delta[row, t, g_of_c]
                out[row] += coef * x[row - t]
        start += n
    return out
