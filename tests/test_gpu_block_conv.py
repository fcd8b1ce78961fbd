"""DFlash2 in-block convolution on the GPU vs the fp64 sequential oracle.

Tolerance from the arithmetic: coef = base + delta is an fp32 sum of two bf16
values, each output accumulates at most `taps` fp32 products in order, and the
result is rounded to bf16 (<= 2^-9 relative).  So
    |got - ref| <= 2^-8 |ref| + 1e-5 * sum_t (|base| + |delta|) |x|
(the second term bounds the fp32 accumulation, the oracle evaluates it on the
absolute values).
"""
import numpy as np
import pytest
import torch

import non_causal_block_amd as nb
import workloads
from gpu_helpers import bf16_tensor, dev
from oracle.block_conv import block_conv_f64

pytestmark = pytest.mark.gpu

CASES = [
    # (block_lens, channels, groups, taps)
    ([5, 16, 1], 256, 8, 16),
    ([16] * 8, 4096, 32, 16),
    ([9, 0, 3], 6, 2, 4),          # 3 channels per group: a channel pair straddles two groups
    ([16, 7], 64, 4, 20),          # more taps than positions
    ([1], 2, 1, 1),
    ([4, 15, 8, 2, 16, 11], 1024, 16, 8),
    ([40, 17, 3, 33], 512, 8, 16),   # blocks longer than the 16-position chunks of the tiled kernel
    ([9, 33], 256, 128, 8),          # more groups than the tiled kernel stages: the per-position kernel
    ([16] * 64, 5120, 32, 16),       # the benchmark's shape (64 requests x 16 positions)
    ([20, 35, 16], 1024, 16, 3),     # odd tap count, two tap pairs, later chunks
    ([18, 5, 0, 31], 768, 12, 7),    # four tap pairs, 64 channels per group
    ([16, 2], 1536, 3, 16),          # 512 channels per group: a workgroup inside one group
    ([16, 5], 5120, 128, 16),        # 128 groups of 40 channels: a workgroup stages 14 of them
    ([12, 16], 64, 32, 6),           # 2 channels per group: one workgroup stages all 32 groups
]


def _f(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_block_conv_matches_sequential_oracle(case):
    blocks, C, G, taps = CASES[case]
    x, base, delta = workloads.block_conv_inputs(blocks, C, G, taps, seed=500 + case)
    d = dev()
    out = nb.block_conv(bf16_tensor(x, d), bf16_tensor(base, d), bf16_tensor(delta, d),
                        torch.tensor(blocks, dtype=torch.int32, device=d), groups=G)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = block_conv_f64(_f(x), _f(base), _f(delta), blocks, G)
    mag = block_conv_f64(np.abs(_f(x)), np.abs(_f(base)), np.abs(_f(delta)), blocks, G)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * mag
    assert np.isfinite(got).all()
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    assert (err <= bound).all(), (case, worst, err[worst], bound[worst])
