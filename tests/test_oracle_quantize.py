"""Pins for the oracle quantiser and dequantiser.

Checked against: a hand-worked 3x32 example (tests/golden), an exactly
representable construction that must round-trip losslessly, the block-amax →
±6 property, and the sign / power-of-two invariances the format implies.
"""

import numpy as np
import pytest

import oracle
from workloads import to_bf16_bits


def _bits(vals):
    return to_bf16_bits(np.array(vals, dtype=np.float32))


def test_hand_worked_example(golden):
    g = golden("quantize_hand_example.txt")
    rows = []
    for r in ("row0", "row1", "row2"):
        rows.append([float(v) for v in g[r]] + [float(v) for v in g[r + "b"]])
    x = _bits(rows)
    # the construction uses only bf16-exact values
    assert np.array_equal(oracle.bf16_bits_to_f32(x), np.array(rows, dtype=np.float32))
    codes, scales, gs = oracle.quantize(x)
    assert gs == np.float32(float(g["g"][0]))
    for i in range(3):
        assert list(scales[i]) == [int(v, 16) for v in g[f"scales{i}"]], i
        assert list(codes[i]) == [int(v, 16) for v in g[f"codes{i}"]], i


def _lossless_case(seed, M=6, K=64, j=-3):
    """x built so every block is exactly representable: x = c·s·2^j, max|c| = 6."""
    rng = np.random.default_rng(seed)
    e2 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    nb = K // 16
    c = rng.choice(e2, size=(M, nb, 16)) * rng.choice([-1, 1], size=(M, nb, 16))
    c[:, :, 0] = 6.0 * rng.choice([-1, 1], size=(M, nb))      # block amax = 6·s·2^j
    # arbitrary normal/subnormal E4M3 scales (bytes 0x01..0x7E), one per block
    s_bytes = rng.integers(1, 0x7F, size=(M, nb))
    s_bytes[0, 0] = 0x7E                                      # the tensor amax block
    s = oracle.e4m3_decode(s_bytes)
    x = c * s[:, :, None] * 2.0 ** j
    return x.reshape(M, K), s_bytes, c.reshape(M, K)


@pytest.mark.parametrize("seed", range(6))
def test_lossless_round_trip(seed):
    x64, s_bytes, c = _lossless_case(seed)
    x = _bits(x64.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f32(x).astype(np.float64), x64)  # bf16-exact
    codes, scales, g = oracle.quantize(x)
    assert g == np.float32(2.0 ** -3)                      # A = 2688·2^j → g = 2^j
    assert np.array_equal(scales, s_bytes.astype(np.uint8))
    back = oracle.dequantize(codes, scales, g)
    assert np.array_equal(back, x64)


def _gaussian(seed, M=64, K=256, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    if outliers:
        pos = rng.choice(x.size, size=max(1, x.size // 1000), replace=False)
        x.reshape(-1)[pos] *= 50
    return _bits(x)


@pytest.mark.parametrize("seed", range(4))
def test_block_amax_maps_to_six(seed):
    x = _gaussian(seed)
    codes, scales, g = oracle.quantize(x)
    c = oracle.unpack_nibbles(codes).reshape(x.shape[0], -1, 16)
    xf = np.abs(oracle.bf16_bits_to_f32(x)).reshape(c.shape)
    amax_pos = xf.argmax(axis=2)
    amax_code = np.take_along_axis(c, amax_pos[:, :, None], axis=2)[:, :, 0]
    normal = scales >= 0x08                                 # S >= 2^-6
    assert np.all((amax_code[normal] & 7) == 7)
    # the block holding the tensor amax gets the top scale 448
    i, k = np.unravel_index(np.argmax(xf.reshape(x.shape)), x.shape)
    assert scales[i, k // 16] == 0x7E


def test_subnormal_scale_block_may_not_reach_six():
    # g = 1; block amax 9·2^-9 → a/6 = 1.5·2^-9, a tie between the E4M3
    # subnormals 0x01 and 0x02 → 0x02 (even) = 2^-8; q = 9·2^-9 · 2^8 = 4.5 → 4
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 2688.0
    x[0, 16] = 0.017578125
    codes, scales, g = oracle.quantize(_bits(x))
    assert g == 1.0 and scales[0, 1] == 0x02
    assert oracle.unpack_nibbles(codes)[0, 16] == 6


@pytest.mark.parametrize("seed", range(3))
def test_sign_symmetry(seed):
    x = _gaussian(seed + 10)
    neg = x ^ np.uint16(0x8000)
    c1, s1, g1 = oracle.quantize(x)
    c2, s2, g2 = oracle.quantize(neg)
    assert g1 == g2 and np.array_equal(s1, s2)
    assert np.array_equal(c1 ^ np.uint8(0x88), c2)


@pytest.mark.parametrize("k", [-20, -5, 3, 17])
def test_power_of_two_invariance(k):
    x = _gaussian(5)
    xf = oracle.bf16_bits_to_f32(x) * np.float32(2.0 ** k)
    xk = _bits(xf)
    c1, s1, g1 = oracle.quantize(x)
    c2, s2, g2 = oracle.quantize(xk)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert g2 == np.float32(g1 * np.float32(2.0 ** k))


def test_all_zero_tensor():
    x = np.zeros((4, 32), np.uint16)
    x[1, 3] = 0x8000                      # a negative zero keeps its sign
    codes, scales, g = oracle.quantize(x)
    assert g == 1.0 and not scales.any()
    want = np.zeros((4, 16), np.uint8)
    want[1, 1] = 0x80                     # element 3 = high nibble of byte 1
    assert np.array_equal(codes, want)


def test_domain_floor():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 2.0 ** -101
    with pytest.raises(ValueError):
        oracle.quantize(_bits(x))
    x[0, 0] = 2.0 ** -100
    codes, scales, g = oracle.quantize(_bits(x))
    assert scales[0, 0] == 0x7E


def test_rows_with_amax_match_full():
    x = _gaussian(21, M=40)
    c, s, g = oracle.quantize(x)
    A = np.abs(oracle.bf16_bits_to_f32(x)).max()
    rows = [0, 7, 39]
    c2, s2, g2 = oracle.quantize(x[rows], amax=A)
    assert g2 == g and np.array_equal(c2, c[rows]) and np.array_equal(s2, s[rows])
    with pytest.raises(ValueError):
        oracle.quantize(x, amax=A / 2)


def test_dequant_error_bounded():
    # |x - deq| <= S·g (half the widest E2M1 step, 4→6), up to the binary32
    # rounding of the reciprocal r = 1/(S·g) near a midpoint
    x = _gaussian(3, outliers=False)
    c, s, g = oracle.quantize(x)
    d = oracle.dequantize(c, s, g)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    step = np.repeat(oracle.e4m3_decode(s), 16, axis=1) * float(g)
    assert np.all(np.abs(xf - d) <= step * (1 + 2.0 ** -20))
    rel = np.linalg.norm(xf - d) / np.linalg.norm(xf)
    assert 0.02 < rel < 0.15
