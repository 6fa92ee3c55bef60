"""GPU parity of the two-dimensional 16x16 weight blocks (NVFP4_Q_BLOCK_2D)
against the oracle (reading R25; source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成",
二、方法 / NVFP4 训练的工程细节, weight blocks along two dimensions).

Codes, scales and the tensor scale must be bit-exact.  The GEMM takes such
weights unchanged (the scales keep the [N, K/16] layout); its output is held
to the same bound as with 1-D weights.
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import (GEMM_TOL, announce, bf16_to_dev, f32_to_dev, gemm_errors, to_bits, to_np,
                         u8_to_dev)

pytestmark = pytest.mark.gpu


def _check(x_bits):
    M, K = x_bits.shape
    announce(f"quantize 2-D M={M} K={K}")
    c, s, g = nv.quantize(bf16_to_dev(x_bits), blocks2d=True)
    torch.cuda.synchronize()
    rc, rs, rg = oracle.quantize(x_bits, blocks2d=True)
    assert to_np(g)[0] == rg
    assert np.array_equal(to_np(s), rs)
    assert np.array_equal(to_np(c), rc)


@pytest.mark.parametrize("M,K,seed", [(300, 416, 1), (16, 32, 2), (1, 32, 3), (17, 64, 4),
                                      (257, 3072, 5), (33, 14336, 6)])
def test_blocks2d_bit_exact(M, K, seed):
    _check(workloads.random_matrix(seed, M, K, 0.02, outliers=True))


def test_blocks2d_qkv_weight_full_size():
    # the QKV projection's weight [9216, 3072], as quantised once offline
    _check(workloads.qkv().w)


def test_blocks2d_edge_values():
    x = workloads.random_matrix(7, 48, 64, 1.0)
    x[:16, :16] = 0                                   # a zero tile: scale 0, codes +0
    x[16, 20] = 0x7F7F                                # the largest finite bf16 in one tile
    x[40:, 48:] = 0x8000                              # -0.0: keeps its sign
    _check(x)


def test_gemm_with_2d_weights():
    M, N, K = 300, 290, 416
    announce(f"gemm with 2-D weights M={M} N={N} K={K}")
    x = workloads.random_matrix(11, M, K, 1.0, outliers=True)
    w = workloads.random_matrix(12, N, K, 0.02)
    qa, qw = oracle.quantize(x), oracle.quantize(w, blocks2d=True)
    c64, cref = oracle.gemm_ref(*qa, *qw)
    wq = nv.quantize(bf16_to_dev(w), blocks2d=True)
    out = nv.gemm(u8_to_dev(qa[0]), u8_to_dev(qa[1]), f32_to_dev(qa[2]), *wq)
    torch.cuda.synchronize()
    e_ref, e_64 = gemm_errors(to_bits(out), c64, cref)
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL, (e_ref, e_64)


def test_transpose_on_gpu():
    # the property 2-D blocks exist for, on the GPU's own bytes: Wᵀ gets the
    # transposed codes and, per tile, the same scale byte
    M, K = 64, 96
    w = workloads.random_matrix(13, M, K, 0.02, outliers=True)
    c, s, g = [to_np(t) for t in nv.quantize(bf16_to_dev(w), blocks2d=True)]
    ct, st, gt = [to_np(t) for t in nv.quantize(bf16_to_dev(np.ascontiguousarray(w.T)), blocks2d=True)]
    torch.cuda.synchronize()

    def nibbles(b, rows, cols):          # element 2j in the low nibble of byte j
        return np.stack([b & 0xF, b >> 4], axis=-1).reshape(rows, cols)

    assert g[0] == gt[0]
    assert np.array_equal(nibbles(c, M, K), nibbles(ct, K, M).T)
    tiles = s[::16, :]                   # [M/16, K/16]: the scale of each tile
    tiles_t = st[::16, :]                # [K/16, M/16]
    assert np.array_equal(tiles, tiles_t.T)
