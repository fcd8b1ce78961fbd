"""Pins of the bidirectional-span (mm-prefix) extension of the oracle.

Reading: in a causal request, two positions inside one listed span [s, e) see
each other in both directions (a multimodal prefix is attended as a whole),
everything else stays causal; non-causal requests see every key anyway.

* A visibility table written by hand.
* The oracle (high end extended to the span's end) against the pure-Python
  brute force (same-span rule), random spans, windows and flags.
* Invariants, bitwise in the oracle: spans that end inside the context change
  nothing for block queries; a span covering the whole block makes a causal
  request equal to the non-causal one; spans do not touch non-causal requests;
  one-position spans change nothing.
"""
import numpy as np
import pytest

import oracle
from oracle import brute


def _bits(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _f(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_hand_written_visibility():
    # L = 4, n = 4, causal, one span covering positions 5 and 6
    want = np.array([
        [1, 1, 1, 1, 1, 0, 0, 0],   # p = 4: outside the span -> keys 0..4
        [1, 1, 1, 1, 1, 1, 1, 0],   # p = 5: in [5, 7) -> also key 6
        [1, 1, 1, 1, 1, 1, 1, 0],   # p = 6: in [5, 7) -> keys 0..6
        [1, 1, 1, 1, 1, 1, 1, 1],   # p = 7: outside -> keys 0..7
    ], dtype=bool)
    assert np.array_equal(brute.mask_matrix(4, 4, True, 0, [(5, 7)]), want)
    # the window still bounds the low side: W = 2
    want_w = np.zeros_like(want)
    for i, (lo, hi) in enumerate([(3, 4), (4, 6), (5, 6), (6, 7)]):
        want_w[i, lo:hi + 1] = True
    assert np.array_equal(brute.mask_matrix(4, 4, True, 2, [(5, 7)]), want_w)


def _random_case(rng, B=3):
    ctx = rng.integers(0, 12, size=B)
    blk = rng.integers(0, 6, size=B)
    spans = []
    for r in range(B):
        T, lst, pos = int(ctx[r] + blk[r]), [], 0
        while pos < T:
            s = int(pos + rng.integers(0, 4))
            if s >= T:
                break
            e = min(T, int(s + rng.integers(1, 5)))
            lst.append((s, e))
            pos = e
        spans.append(lst)
    return ctx, blk, spans


@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_brute_force_with_spans(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = 4, 2, 8
    for _ in range(5):
        ctx, blk, spans = _random_case(rng)
        c = rng.integers(0, 2, size=3).astype(np.uint8)
        W = int(rng.choice([0, 0, 3, 7]))
        tq, tk = int(blk.sum()), int((ctx + blk).sum())
        q, k, v = _bits(rng, (tq, Hq, D)), _bits(rng, (tk, Hkv, D)), _bits(rng, (tk, Hkv, D))
        a = oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, W, 0.35, spans=spans)
        b = brute.block_attn(_f(q), _f(k), _f(v), ctx, blk, c, Hq, Hkv, D, W, 0.35, spans=spans)
        assert np.abs(a - b).max(initial=0.0) <= 1e-12


def _case(seed=11):
    rng = np.random.default_rng(seed)
    ctx = np.array([20, 7, 13], dtype=np.int32)
    blk = np.array([9, 5, 16], dtype=np.int32)
    Hq, Hkv, D = 4, 2, 16
    tq, tk = int(blk.sum()), int((ctx + blk).sum())
    return ctx, blk, Hq, Hkv, D, _bits(rng, (tq, Hq, D)), _bits(rng, (tk, Hkv, D)), _bits(rng, (tk, Hkv, D))


def test_spans_inside_the_context_change_nothing_for_block_queries():
    ctx, blk, Hq, Hkv, D, q, k, v = _case()
    c = np.ones(3, dtype=np.uint8)
    base = oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 0, 0.3)
    spans = [[(0, 5), (8, 20)], [(2, 7)], [(1, 3), (5, 13)]]
    assert np.array_equal(oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 0, 0.3, spans=spans), base)


def test_a_span_over_the_whole_block_equals_non_causal():
    ctx, blk, Hq, Hkv, D, q, k, v = _case()
    spans = [[(int(ctx[r]) - 3 if ctx[r] >= 3 else 0, int(ctx[r] + blk[r]))] for r in range(3)]
    causal_span = oracle.block_attn_f64(q, k, v, ctx, blk, np.ones(3, np.uint8), Hq, Hkv, D, 0, 0.3, spans=spans)
    non_causal = oracle.block_attn_f64(q, k, v, ctx, blk, np.zeros(3, np.uint8), Hq, Hkv, D, 0, 0.3)
    assert np.array_equal(causal_span, non_causal)


def test_spans_do_not_touch_non_causal_requests_and_single_positions_do_nothing():
    ctx, blk, Hq, Hkv, D, q, k, v = _case()
    c = np.array([0, 1, 0], dtype=np.uint8)
    base = oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 5, 0.3)
    spans = [[(21, 29)], [(7, 8), (9, 10), (11, 12)], [(13, 29)]]  # request 1: one-position spans only
    assert np.array_equal(oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 5, 0.3, spans=spans), base)


def test_a_span_past_the_request_end_is_clipped_to_its_keys():
    """A span may end past the request's last key T-1 (the ABI clips it); a query
    sees only its own request's keys, so such a span equals the one cut at T, and
    both equal the brute force (which only ever looks at keys 0..T-1)."""
    ctx, blk, Hq, Hkv, D, q, k, v = _case()
    c = np.ones(3, dtype=np.uint8)
    T = ctx + blk
    past = [[(int(ctx[0]) + 2, int(T[0]) + 50)], [(int(ctx[1]), int(T[1]) + 1)], [(0, int(T[2]) + 1000)]]
    cut = [[(s, min(e, int(T[r]))) for s, e in sp] for r, sp in enumerate(past)]
    a = oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 0, 0.3, spans=past)
    assert np.array_equal(a, oracle.block_attn_f64(q, k, v, ctx, blk, c, Hq, Hkv, D, 0, 0.3, spans=cut))
    b = brute.block_attn(_f(q), _f(k), _f(v), ctx, blk, c, Hq, Hkv, D, 0, 0.3, spans=past)
    assert np.abs(a - b).max() <= 1e-12
