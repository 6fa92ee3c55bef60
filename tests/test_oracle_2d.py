"""Pins of the oracle's two-dimensional weight blocks (reading R25: 16x16 tiles,
one E4M3 scale per tile stored on each of its rows).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 训练的工程细节
(weights scaled in blocks along two dimensions, so that W and its transpose
share one quantisation).  The checks do not reuse the oracle's formulas: a
hand-worked tensor, the transpose identity that motivates 2-D blocks, the
reduction to 1-D blocks when the rows of a group are equal, and the tile scale
as the largest row scale of its group (E4M3 rounding is monotone).
"""

import numpy as np
import pytest

import oracle
import workloads
from oracle.formats import bf16_rne_from_f64


def _bits(values):
    return bf16_rne_from_f64(np.asarray(values, dtype=np.float64))


def test_hand_worked_tiles():
    # 32 x 32: row groups {0..15, 16..31} x column blocks {0..15, 16..31}.
    x = np.zeros((32, 32))
    x[3, 5] = 2688.0       # tensor amax 6·448 → g = 1; tile (0,0) amax 2688 → S = 448
    x[9, 1] = -448.0       #   |x|·r = 448/448 = 1   → E2M1 1.0 (bits 010), negative
    x[0, 20] = 6.0         # tile (0,1): amax 6 → S = 1
    x[15, 17] = -1.5       #   1.5 → E2M1 bits 011, negative
    x[7, 31] = 3.0         #   3.0 → E2M1 bits 101
    x[20, 2] = 12.0        # tile (1,0): amax 12 → S = 2
    x[31, 0] = 1.0         #   1/2 = 0.5 → E2M1 bits 001
    x[16, 15] = -0.9       #   0.45 → nearest E2M1 is 0.5 → bits 001, negative
    # tile (1,1) stays zero → S = 0, codes +0
    codes, scales, g = oracle.quantize(_bits(x), blocks2d=True)
    assert g == np.float32(1.0)
    e4m3 = {448.0: 0x7E, 1.0: 0x38, 2.0: 0x40, 0.0: 0x00}
    want_scales = np.zeros((32, 2), dtype=np.uint8)
    want_scales[:16, 0], want_scales[:16, 1] = e4m3[448.0], e4m3[1.0]
    want_scales[16:, 0], want_scales[16:, 1] = e4m3[2.0], e4m3[0.0]
    assert np.array_equal(scales, want_scales)
    nib = oracle.unpack_nibbles(codes)
    want = np.zeros((32, 32), dtype=np.uint8)
    want[3, 5] = 0b0111                      # 2688/448 = 6 → E2M1 6 (111)
    want[9, 1] = 0b1010
    want[0, 20] = 0b0111
    want[15, 17] = 0b1011
    want[7, 31] = 0b0101
    want[20, 2] = 0b0111
    want[31, 0] = 0b0001
    want[16, 15] = 0b1001
    assert np.array_equal(nib, want)


@pytest.mark.parametrize("M,K,seed", [(48, 64, 1), (32, 32, 2), (64, 96, 3)])
def test_transpose_shares_the_quantisation(M, K, seed):
    # the point of 2-D blocks: W and Wᵀ quantise to the same values, transposed
    x = workloads.random_matrix(seed, M, K, 1.0, outliers=True)
    d = oracle.dequantize(*oracle.quantize(x, blocks2d=True))
    dt = oracle.dequantize(*oracle.quantize(np.ascontiguousarray(x.T), blocks2d=True))
    assert np.array_equal(d, dt.T)
    # 1-D blocks do not have this property on the same input
    d1 = oracle.dequantize(*oracle.quantize(x))
    d1t = oracle.dequantize(*oracle.quantize(np.ascontiguousarray(x.T)))
    assert not np.array_equal(d1, d1t.T)


@pytest.mark.parametrize("M", [16, 37])
def test_equal_rows_reduce_to_1d(M):
    # when every row of a 16-row group is the same, each tile's amax is the
    # row's block amax: the 2-D result is the 1-D one
    base = workloads.random_matrix(4, (M + 15) // 16, 64, 1.0, outliers=True)
    x = np.repeat(base, 16, axis=0)[:M]
    q1, q2 = oracle.quantize(x), oracle.quantize(x, blocks2d=True)
    for a, b in zip(q1, q2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M,K,seed", [(50, 64, 5), (16, 32, 6), (1, 48, 7)])
def test_tile_scale_is_the_largest_row_scale(M, K, seed):
    x = workloads.random_matrix(seed, M, K, 1.0, outliers=True)
    _, s1, g1 = oracle.quantize(x)
    _, s2, g2 = oracle.quantize(x, blocks2d=True)
    assert g1 == g2
    for r0 in range(0, M, 16):
        grp = s1[r0:r0 + 16]
        assert np.array_equal(s2[r0:r0 + 16], np.broadcast_to(grp.max(axis=0), grp.shape))


def test_options_exclude_each_other():
    x = workloads.random_matrix(8, 16, 32, 1.0)
    with pytest.raises(ValueError):
        oracle.quantize(x, adaptive46=True, blocks2d=True)
    with pytest.raises(ValueError):
        oracle.quantize(x, amax=10.0, blocks2d=True)
