"""Pins of the DFlash2 block-convolution oracle (oracle/block_conv.py).

* A case worked by hand (3 positions, 4 channels in 2 groups, 2 taps).
* delta = 0 reduces to a per-channel causal convolution inside each block:
  numpy's convolve, truncated at the block (taps never cross into the previous
  request's block).
* Blocks are independent: changing one request's x leaves the others' outputs.
* One tap: out = (base[0] + delta[:, 0, g]) * x.
* Taps beyond the block length contribute nothing.
"""
import numpy as np
import pytest

from oracle.block_conv import block_conv_f64


def test_hand_worked_example():
    x = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]], dtype=np.float64)
    base = np.array([[1, 0, 2, 0], [0, 1, 0, 1]], dtype=np.float64)           # [taps=2, C=4]
    delta = np.array([[[0, 0], [0, 0]],                                        # i = 0: [t][g]
                      [[1, 0], [0, 2]],                                        # i = 1
                      [[0, 1], [1, 0]]], dtype=np.float64)                     # i = 2
    # channels 0,1 -> group 0; channels 2,3 -> group 1
    # i=0: t=0 coef [1,0,2,0]                   * x0 [1,2,3,4]  = [1,0,6,0]
    # i=1: t=0 coef [1,0,2,0]+[1,1,0,0]=[2,1,2,0] * x1 = [10,6,14,0]
    #      t=1 coef [0,1,0,1]+[0,0,2,2]=[0,1,2,3] * x0 = [0,2,6,12]  -> [10,8,20,12]
    # i=2: t=0 coef [1,0,2,0]+[0,0,1,1]=[1,0,3,1] * x2 = [9,0,33,12]
    #      t=1 coef [0,1,0,1]+[1,1,0,0]=[1,2,0,1] * x1 = [5,12,0,8]  -> [14,12,33,20]
    want = np.array([[1, 0, 6, 0], [10, 8, 20, 12], [14, 12, 33, 20]], dtype=np.float64)
    assert np.array_equal(block_conv_f64(x, base, delta, [3], groups=2), want)


def test_zero_delta_is_a_causal_convolution_inside_each_block():
    rng = np.random.default_rng(0)
    blocks = [5, 1, 9, 0, 7]
    C, taps = 6, 4
    x = rng.standard_normal((sum(blocks), C))
    base = rng.standard_normal((taps, C))
    out = block_conv_f64(x, base, np.zeros((sum(blocks), taps, 3)), blocks, groups=3)
    start = 0
    for n in blocks:
        for c in range(C if n else 0):
            want = np.convolve(x[start:start + n, c], base[:, c])[:n]
            assert np.allclose(out[start:start + n, c], want, rtol=0, atol=1e-12)
        start += n


def test_blocks_are_independent():
    rng = np.random.default_rng(1)
    blocks = [4, 6, 3]
    C, G, taps = 8, 4, 5
    x = rng.standard_normal((13, C))
    base = rng.standard_normal((taps, C))
    delta = rng.standard_normal((13, taps, G))
    a = block_conv_f64(x, base, delta, blocks, G)
    x2 = x.copy()
    x2[4:10] += 7.0  # the second request only
    b = block_conv_f64(x2, base, delta, blocks, G)
    assert np.array_equal(a[:4], b[:4]) and np.array_equal(a[10:], b[10:])
    assert not np.allclose(a[4:10], b[4:10])


def test_single_tap_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 12))
    base = rng.standard_normal((1, 12))
    delta = rng.standard_normal((7, 1, 3))
    g = np.arange(12) // 4
    want = (base[0][None, :] + delta[:, 0, g]) * x
    assert np.allclose(block_conv_f64(x, base, delta, [3, 4], groups=3), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("extra", [1, 5])
def test_taps_past_the_block_do_nothing(extra):
    rng = np.random.default_rng(3)
    blocks = [4, 2]
    C, G = 4, 2
    x = rng.standard_normal((6, C))
    base = rng.standard_normal((4 + extra, C))
    delta = rng.standard_normal((6, 4 + extra, G))
    assert np.array_equal(block_conv_f64(x, base, delta, blocks, G),
                          block_conv_f64(x, base[:4], delta[:, :4], blocks, G))
