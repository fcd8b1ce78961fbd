"""The split-invariance error model (tests/error_model.py), checked on the CPU.

A numpy simulation of the GPU path's rounding steps -- softmax weights rounded to bf16
against each piece's own reference maximum (its first 32-key tile), the denominator
summing the same rounded weights, bf16 normalised partials, a merge of the pieces, a
bf16 output -- for several splits of each request's keys must stay within the
model's per-element bound of the unsplit result, and the bound must stay a few bf16
ulps of the output, below the parity bound on the largest error (2e-2).
"""
import numpy as np

import oracle
import workloads
from tests import error_model


def _bf16(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _simulate(wl, cuts_for):
    """Output of the rounding model with request r's visible keys cut at cuts_for(r, T)."""
    G = wl.Hq // wl.Hkv
    q = workloads.bf16_bits_to_f32(wl.q).astype(np.float64)
    k = workloads.bf16_bits_to_f32(wl.k).astype(np.float64)
    v = workloads.bf16_bits_to_f32(wl.v).astype(np.float64)
    out = np.zeros((wl.total_q, wl.Hq, wl.D))
    for r in range(wl.B):
        L, n = int(wl.ctx_lens[r]), int(wl.block_lens[r])
        T = L + n
        cuts = [0] + sorted(set(cuts_for(r, T))) + [T]
        for i in range(n):
            p_pos = L + i
            hi = p_pos if wl.causal[r] else T - 1
            for h in range(wl.Hq):
                g = h // G
                z = (k[wl.kv_start[r]:wl.kv_start[r] + T, g] @ q[wl.q_start[r] + i, h]) * wl.scale
                parts = []
                for a, b in zip(cuts[:-1], cuts[1:]):
                    b = min(b, hi + 1)
                    if a >= b:
                        continue
                    ref_max = z[a:min(a + 32, b)].max()        # the piece's first tile
                    w = _bf16(np.exp(z[a:b] - ref_max))
                    o = _bf16(w @ v[wl.kv_start[r] + a:wl.kv_start[r] + b, g] / w.sum())
                    parts.append((ref_max + np.log(w.sum()), o))
                M = max(s for s, _ in parts)
                ws = np.array([np.exp(s - M) for s, _ in parts])
                out[wl.q_start[r] + i, h] = _bf16(sum(wgt * o for wgt, (_, o) in zip(ws, parts)) / ws.sum())
    return out


def test_simulated_splits_stay_within_the_bound():
    wl = workloads.build(3, 4, 2, 64, [300, 170, 500], [9, 5, 9], [0, 1, 0], seed=12, poison=False)
    ref = oracle.run_workload(wl)
    bound = error_model.split_bound(ref, error_model.split_sigma(wl))
    base = _simulate(wl, lambda r, T: [])
    assert np.abs(base - ref).max() <= 2e-2
    rng = np.random.default_rng(3)
    for trial in range(4):
        cut = lambda r, T: sorted(rng.integers(1, T, size=int(rng.integers(1, 8))).tolist())  # noqa: E731
        got = _simulate(wl, cut)
        excess = np.abs(got - base) - bound
        assert excess.max() <= 0, (trial, float(excess.max()))
    # the bound is a few bf16 ulps of the output: its median is under 4% of the output's
    # RMS (one ulp is 2^-8..2^-7 of a value), and no element's bound reaches the parity
    # bound on the largest error (2e-2)
    rms = float(np.sqrt(np.mean(ref * ref)))
    assert np.median(bound) <= 0.04 * rms and bound.max() < 2e-2


def test_sigma_scales_like_the_rounding_of_one_weight():
    # one visible key: the weight is exactly 1 (no rounding error), so sigma is v's own term
    wl = workloads.build(1, 2, 1, 16, [0], [1], [1], seed=4, poison=False)
    sig = error_model.split_sigma(wl)
    v0 = workloads.bf16_bits_to_f32(wl.v).astype(np.float64)[0, 0]
    want = 2.0 ** -8 / np.sqrt(3.0) * np.abs(v0)
    assert np.allclose(sig[0, 0], want, rtol=1e-12) and np.allclose(sig[0, 1], want, rtol=1e-12)
