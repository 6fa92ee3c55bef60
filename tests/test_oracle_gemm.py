"""Pins for the oracle W4A4 GEMM and its epilogue.

Checked against: exact rational arithmetic (fractions.Fraction) on tiny,
non-square shapes (a transposed operand or a wrong scale index fails it), the
unit-scale special case against torch.matmul in float64, exact linearity in
the global scales, the per-block sum form of the dequant equation, and
torch's tanh-form GELU.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.nvfp4 import gemm_exact_fraction
from workloads import random_matrix


def _q(seed, rows, K, sigma=1.0):
    return oracle.quantize(random_matrix(seed, rows, K, sigma))


@pytest.mark.parametrize("M,N,K", [(3, 5, 32), (4, 2, 48), (1, 7, 16)])
def test_gemm_vs_fraction(M, N, K):
    Aq, As, Ag = _q(M * 100 + K, M, K)
    Wq, Ws, Wg = _q(N * 100 + K + 1, N, K, 0.02)
    c64, cb = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg)
    exact = gemm_exact_fraction(Aq, As, Ag, Wq, Ws, Wg)
    for i in range(M):
        for j in range(N):
            e = float(exact[i][j])
            assert abs(c64[i, j] - e) <= 1e-13 * max(1e-30, abs(e)) + 1e-300, (i, j)
    # the bf16 output is one nearest-even rounding of the exact value
    ex = np.array([[float(v) for v in r] for r in exact])
    assert np.array_equal(cb, oracle.bf16_rne_from_f64(ex))


def test_unit_scales_equal_plain_matmul(golden):
    mags = np.array([float(v) for v in golden("e2m1_values.txt")["magnitudes"]])
    rng = np.random.default_rng(5)
    M, N, K = 9, 11, 64
    ca = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    A = np.where(ca & 8, -1.0, 1.0) * mags[ca & 7]
    W = np.where(cw & 8, -1.0, 1.0) * mags[cw & 7]
    ones_a = np.full((M, K // 16), 0x38, np.uint8)        # E4M3 1.0
    ones_w = np.full((N, K // 16), 0x38, np.uint8)
    c64, _ = oracle.gemm_ref(oracle.pack_nibbles(ca), ones_a, np.float32(1),
                             oracle.pack_nibbles(cw), ones_w, np.float32(1))
    ref = torch.matmul(torch.from_numpy(A), torch.from_numpy(W).T).numpy()
    assert np.array_equal(c64, ref)


def test_global_scale_linearity():
    Aq, As, Ag = _q(1, 16, 64)
    Wq, Ws, Wg = _q(2, 24, 64, 0.02)
    c1, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg)
    c2, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, np.float32(Wg * 2))
    assert np.array_equal(c2, 2 * c1)


def test_block_sum_form():
    # Σ_b sA·sW·(Σ_k cA·cW)·gA·gW equals the dequantised product
    Aq, As, Ag = _q(3, 8, 96)
    Wq, Ws, Wg = _q(4, 6, 96, 0.02)
    c64, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg)
    mags = oracle.E2M1_VALUES
    ca, cw = oracle.unpack_nibbles(Aq), oracle.unpack_nibbles(Wq)
    va = np.where(ca & 8, -1.0, 1.0) * mags[ca & 7]
    vw = np.where(cw & 8, -1.0, 1.0) * mags[cw & 7]
    sa, sw = oracle.e4m3_decode(As), oracle.e4m3_decode(Ws)
    out = np.zeros((8, 6))
    for b in range(96 // 16):
        part = va[:, 16 * b:16 * b + 16] @ vw[:, 16 * b:16 * b + 16].T   # exact integers/halves
        out += part * sa[:, b][:, None] * sw[:, b][None, :]
    out *= float(Ag) * float(Wg)
    assert np.allclose(out, c64, rtol=1e-13, atol=0)


def test_bias_is_added():
    Aq, As, Ag = _q(6, 5, 32)
    Wq, Ws, Wg = _q(7, 4, 32, 0.02)
    bias = random_matrix(8, 1, 4, 0.01)[0]
    c0, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg)
    c1, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg, bias_bits=bias)
    b = oracle.bf16_bits_to_f32(bias).astype(np.float64)
    assert np.allclose(c1 - c0, np.broadcast_to(b, c0.shape), rtol=0, atol=1e-15)


def test_gelu_tanh():
    y = np.linspace(-12, 12, 2001)
    g = oracle.gelu_tanh(y)
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(g - oracle.gelu_tanh(-y), y, rtol=1e-14, atol=1e-14)
    assert abs(oracle.gelu_tanh(np.array([20.0]))[0] - 20.0) < 1e-12


def test_gemm_gelu_flag():
    Aq, As, Ag = _q(9, 6, 64)
    Wq, Ws, Wg = _q(10, 5, 64, 0.02)
    c0, _ = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg)
    c1, b1 = oracle.gemm_ref(Aq, As, Ag, Wq, Ws, Wg, gelu=True)
    assert np.array_equal(c1, oracle.gelu_tanh(c0))
    assert np.array_equal(b1, oracle.bf16_rne_from_f64(c1))
