"""Per-element error scale of the GPU path's split-dependent rounding (test infrastructure).

bf16 keeps 8 significant bits, so rounding to nearest has unit roundoff u = 2^-8: a value
x in [2^e, 2^(e+1)) moves by at most half its spacing 2^(e-7), i.e. by a relative error
|e| <= u (reached at the bottom of the binade; 2^-9 at its top).  Taking the absolute
error as uniform over that half-spacing, the relative error's mean square is at most
u^2 / 3.

The kernels round the softmax weights of a key tile to bf16 relative to a per-row
reference maximum, and the denominator sums the same rounded weights (R16), so an output
element is  o_d = sum_j p~_j v_jd / sum_j p~_j  with  p~_j = p_j (1 + e_j).  To first
order the error is
    sum_j p_j e_j (v_jd - o_d) / W,      W = sum_j p_j,
a sum of independent rounding errors whose standard deviation is at most
u / sqrt(3) * sqrt(sum_j p_j^2 (v_jd - o_d)^2) / W.  Which weights round which way
depends on the reference maximum, i.e. on how the keys were split over workgroups.  A
split unit's pieces are also stored as bf16 normalised partials (R11): piece s contributes
(sum_{j in s} p_j v_jd) / W  with a relative rounding error of at most u, again
independent across pieces; for values drawn independently of the keys the expected
square of a piece's contribution is sum_{j in s} p_j^2 v_jd^2 / W^2, so the partials add
at most  u / sqrt(3) * sqrt(sum_j p_j^2 v_jd^2) / W  of standard deviation.  The final
bf16 rounding of each output moves it by at most u |o_d|, so two splits' outputs differ
by at most 2 u |o_d| = 2^-7 |o_d| from that.  Hence the per-element bound

    |A_d - B_d| <= 2^-7 |o_d| + k * sqrt(2) * sigma_d + 1e-6,
    sigma_d = 2^-8 / sqrt(3) * sqrt(sum_j p_j^2 ((v_jd - o_d)^2 + v_jd^2)) / W,

for two splits A and B (sqrt(2): their rounding errors are independent), k standard
deviations (k = 7: with ~10^6 elements a Gaussian tail beyond 7 sigma is ~10^-6 likely),
and 1e-6 for fp32 accumulation in a different order.

``split_sigma`` evaluates sigma_d in float64 from the workload's bf16 inputs.
"""
from __future__ import annotations

import numpy as np

import workloads


def split_sigma(wl: workloads.Workload) -> np.ndarray:
    """sigma_d for every output element: float64 [total_q, Hq, D]."""
    G = wl.Hq // wl.Hkv
    q = workloads.bf16_bits_to_f32(wl.q).astype(np.float64)
    k = workloads.bf16_bits_to_f32(wl.k).astype(np.float64)
    v = workloads.bf16_bits_to_f32(wl.v).astype(np.float64)
    sig = np.zeros((wl.total_q, wl.Hq, wl.D))
    qs, ks = wl.q_start, wl.kv_start
    for r in range(wl.B):
        L, n = int(wl.ctx_lens[r]), int(wl.block_lens[r])
        if n == 0:
            continue
        T = L + n
        pos = L + np.arange(n)
        keys = np.arange(T)
        vis = np.ones((n, T), dtype=bool)
        if wl.causal[r]:
            vis &= keys[None, :] <= pos[:, None]
        if wl.window > 0:
            vis &= keys[None, :] >= (pos - wl.window + 1)[:, None]
        for g in range(wl.Hkv):
            K = k[ks[r]:ks[r] + T, g]
            V = v[ks[r]:ks[r] + T, g]
            Q = q[qs[r]:qs[r] + n, g * G:(g + 1) * G].reshape(n * G, wl.D)
            z = (Q @ K.T) * wl.scale
            m = np.repeat(vis, G, axis=0)
            z = np.where(m, z, -np.inf)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            W = p.sum(axis=1, keepdims=True)
            o = (p @ V) / W
            p2 = p * p
            s_v2 = p2 @ (V * V)
            s_v = p2 @ V
            s_1 = p2.sum(axis=1, keepdims=True)
            centred = s_v2 - 2.0 * o * s_v + o * o * s_1
            var = np.maximum(centred, 0.0) + s_v2
            sig[qs[r]:qs[r] + n, g * G:(g + 1) * G] = (2.0 ** -8 / np.sqrt(3.0) * np.sqrt(var) / W).reshape(n, G, wl.D)
    return sig


def split_bound(ref: np.ndarray, sigma: np.ndarray, k: float = 7.0) -> np.ndarray:
    """Largest |A - B| two splits may show per element (ref: the exact output)."""
    return 2.0 ** -7 * np.abs(ref) + k * np.sqrt(2.0) * sigma + 1e-6
