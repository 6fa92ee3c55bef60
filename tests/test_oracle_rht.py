"""Pins for the oracle's random Hadamard transform and the quantised
weight-gradient operands (oracle/rht.py).

Each pin is independent of the module's own construction: the Hadamard matrix
against scipy's, the transform against an exact rational brute force that
builds H from the bit formula, the hand-worked example in
tests/golden/rht_hand_example.txt, the inverse transform, the invariance of
the weight-gradient contraction, and the evening-out the pages give as the
transform's purpose (a spike spreads flat; heavy tails approach the normal
kurtosis).
"""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from workloads import to_bf16_bits


def _popcount(v):
    return bin(v).count("1")


def _bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def _hex_row(vals):
    return np.array([int(v, 16) for v in vals], dtype=np.uint8)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64])
def test_hadamard_is_sylvester(n):
    h = oracle.hadamard(n)
    assert np.array_equal(h, scipy.linalg.hadamard(n).astype(np.float64))
    assert np.array_equal(h @ h.T, n * np.eye(n))


def test_hand_example(golden):
    g = golden("rht_hand_example.txt")
    T, N = int(g["T"][0]), int(g["N"][0])
    mask = int(g["sign_mask"][0], 16)
    x = np.zeros((T, N), dtype=np.float32)
    for item in g["nonzero_inputs"]:
        t, n, v = item.split(",")
        x[int(t), int(n)] = float(v)
    x[16:32, 1] = float(g["constant_column_1_group_1"][0])
    xb = _bits(x)
    y = oracle.rht(xb, mask)
    assert np.array_equal(y[16:32, 1], np.array([float(v) for v in g["transformed_col1_group1"]],
                                                dtype=np.float32))
    codes, scales, gs = oracle.quantize_rht(xb, mask)
    assert np.float32(gs).view(np.uint32) == int(g["g_bits"][0], 16)
    for n in range(N):
        assert np.array_equal(codes[n], _hex_row(g[f"codes_row{n}"])), n
        assert np.array_equal(scales[n], _hex_row(g[f"scales_row{n}"])), n


@pytest.mark.parametrize("seed,mask", [(1, 0x0000), (2, 0xFFFF), (3, 0x8421), (4, 0x5A3C)])
def test_exact_rational_brute_force(seed, mask):
    rng = np.random.default_rng(seed)
    T, N = 32, 3
    xb = _bits(rng.standard_normal((T, N)) * np.exp2(rng.integers(-8, 8, (T, N))))
    xf = oracle.bf16_bits_to_f32(xb)
    y = oracle.rht(xb, mask)
    for n in range(N):
        for t in range(T):
            gr, i = divmod(t, 16)
            acc = Fraction(0)
            for k in range(16):
                h = -1 if _popcount(i & k) & 1 else 1
                s = -1 if (mask >> k) & 1 else 1
                acc += h * s * Fraction(float(xf[16 * gr + k, n]))
            assert y[t, n] == np.float32(float(acc / 4)), (t, n)


def test_inverse_recovers_input():
    rng = np.random.default_rng(5)
    mask = 0x3C5A
    x = oracle.bf16_bits_to_f32(_bits(rng.standard_normal((64, 7)))).astype(np.float64)
    y = oracle.rht_f64(x, mask)
    s = np.array([-1.0 if (mask >> k) & 1 else 1.0 for k in range(16)])
    h = scipy.linalg.hadamard(16).astype(np.float64)
    inv = np.diag(s) @ h.T / 4.0                          # Rᵀ = diag(s)·Hᵀ/4
    back = np.einsum("ik,gkn->gin", inv, y.reshape(4, 16, 7)).reshape(64, 7)
    assert np.array_equal(back, x)


def test_contraction_is_invariant():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((96, 5))
    b = rng.standard_normal((96, 4))
    for mask in (0, 0xFFFF, 0x1234):
        lhs = oracle.rht_f64(a, mask).T @ oracle.rht_f64(b, mask)
        assert np.allclose(lhs, a.T @ b, rtol=1e-12, atol=1e-12)
    # two different sign masks do not cancel
    lhs = oracle.rht_f64(a, 0x0001).T @ oracle.rht_f64(b, 0x0000)
    assert not np.allclose(lhs, a.T @ b, rtol=1e-3, atol=1e-3)


def test_constant_group_goes_to_first_output():
    # a column constant along the 16 tokens of a group: H·1 = 16·e_0, so only the
    # group's first output is non-zero (4c with every sign +1); varying along N
    # does not matter, which a transform along the wrong axis would break
    c = np.array([1.0, -2.5, 0.75, 3.0], dtype=np.float32)
    x = np.tile(c, (32, 1))
    y = oracle.rht(_bits(x), 0)
    assert np.array_equal(y[0], 4 * c) and np.array_equal(y[16], 4 * c)
    assert not y[1:16].any() and not y[17:32].any()


def test_quantize_f32_equals_quantize_on_bf16_values():
    rng = np.random.default_rng(7)
    xb = _bits(rng.standard_normal((9, 64)) * 3)
    for mode in ({}, {"adaptive46": True}, {"blocks2d": True}):
        got = oracle.quantize_f32(oracle.bf16_bits_to_f32(xb), **mode)
        ref = oracle.quantize(xb, **mode)
        assert all(np.array_equal(a, b) for a, b in zip(got, ref)), mode


def test_spike_is_spread_flat():
    # one non-zero per group: every output of the group has magnitude |x|/4
    # (the transform evens out a block whose energy sits in one element)
    x = np.zeros((32, 5), dtype=np.float32)
    x[3, 0], x[7, 1], x[16, 2], x[31, 3], x[20, 4] = 8.0, -3.0, 0.5, 12.0, -1.25
    y = oracle.rht(_bits(x), 0xA5C3)
    for n, (t, v) in enumerate([(3, 8.0), (7, -3.0), (16, 0.5), (31, 12.0), (20, -1.25)]):
        g = t // 16
        assert np.array_equal(np.abs(y[16 * g:16 * g + 16, n]), np.full(16, abs(v) / 4, np.float32))
        assert not np.delete(y[:, n], np.s_[16 * g:16 * g + 16]).any()


def test_heavy_tails_become_closer_to_normal():
    # Student-t (5 degrees of freedom, kurtosis 9): a sum of 16 independent such
    # values with signs has kurtosis 3 + 6/16; the transform brings the sample
    # kurtosis from about 9 down to about 3.4
    rng = np.random.default_rng(8)
    x = _bits(rng.standard_t(5, (4096, 64)))
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64).ravel()
    y = oracle.rht(x, 0x9D2B).astype(np.float64).ravel()
    kurt = lambda v: np.mean((v - v.mean()) ** 4) / np.var(v) ** 2
    assert kurt(xf) > 6.0 and abs(kurt(y) - 3.375) < 0.3, (kurt(xf), kurt(y))
    assert np.isclose(np.sum(y * y), np.sum(xf * xf), rtol=1e-6)   # energy kept (orthogonal)


def test_exact_zeros_are_positive():
    # zero groups (+0 and -0 inputs) under a mask that flips every sign, and a
    # group whose transform cancels exactly: every zero output is +0 and
    # encodes as code 0, not 0x8
    x = np.zeros((32, 3), dtype=np.float32)
    x[:16, 1] = -0.0
    x[16:32, 2] = np.r_[1.0, 1.0, np.zeros(14)]           # H·x has zeros at odd i
    xb = _bits(x)
    y = oracle.rht(xb, 0xFFFF)
    zero = y == 0
    assert zero.sum() > 60 and not np.signbit(y[zero]).any()
    codes, scales, _ = oracle.quantize_rht(xb, 0xFFFF)
    assert not codes[:2].any() and not scales[:2].any()
    nib = oracle.unpack_nibbles(codes[2:3])[0, 16:32]
    assert np.array_equal(nib[1::2], np.zeros(8, np.uint8))


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        oracle.quantize_rht(np.zeros((48, 4), dtype=np.uint16), 0)      # T not a multiple of 32
    with pytest.raises(ValueError):
        oracle.rht(np.zeros((16, 4), dtype=np.uint16), 1 << 16)         # 17-bit mask
    x = np.zeros((16, 1), dtype=np.float32)
    x[0, 0], x[1, 0] = 2.0 ** 40, 2.0 ** -2                             # a span of 2^42
    with pytest.raises(ValueError):
        oracle.rht(_bits(x), 0)
    x[1, 0] = 2.0 ** 0                                                  # 2^40: exact
    assert oracle.rht(_bits(x), 0)[1, 0] == np.float32((2.0 ** 40 - 1) / 4)
