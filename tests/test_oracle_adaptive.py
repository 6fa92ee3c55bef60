"""Pins of the oracle's adaptive {4, 6} block-scale selection.

Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座
(adaptive scale selection for the KV cache) and the distillation paragraph of
二、方法 (amax target set {4, 6}); the selection rule is the reading stated in
the oracle (smaller binary32 block squared error, ties to 6).
"""

from fractions import Fraction

import numpy as np

import oracle
from workloads import random_matrix, to_bf16_bits


def _row(g, keys):
    return [float(v) for k in keys for v in g[k]]


def test_hand_example(golden):
    g = golden("quantize_adaptive_hand_example.txt")
    x = to_bf16_bits(np.array([_row(g, ("x0", "x1", "x2", "x3"))], dtype=np.float32))
    for adaptive, sk, ck in ((False, "scales_std", "codes_std"), (True, "scales_ad", "codes_ad")):
        codes, scales, gs = oracle.quantize(x, adaptive46=adaptive)
        assert gs == np.float32(float(g["g"][0]))
        assert list(scales[0]) == [int(v, 16) for v in g[sk]], sk
        assert list(codes[0]) == [int(v, 16) for v in g[ck]], ck


def test_hand_example_errors(golden):
    # the binary32 block error of the hand-derived encodings
    g = golden("quantize_adaptive_hand_example.txt")
    xf = np.array(_row(g, ("x1", "x2")), dtype=np.float32).reshape(1, 2, 16)
    neg = np.signbit(xf)
    S6 = np.array([[0x33, 0x38]], dtype=np.uint8)
    S4 = np.array([[0x38, 0x3C]], dtype=np.uint8)
    m6 = np.array([[[7, 6, 5, 4, 3, 1, 0, 7, 6, 5, 4, 3, 1, 0, 0, 0],
                    [7, 5, 3, 1] + [0] * 12]], dtype=np.uint8)
    m4 = np.array([[[6, 5, 4, 3, 2, 1, 0, 6, 5, 4, 3, 2, 1, 0, 0, 0],
                    [6, 4, 2, 1] + [0] * 12]], dtype=np.uint8)
    e6 = oracle.block_sq_error(xf, S6, m6, neg, np.float32(1.0))
    e4 = oracle.block_sq_error(xf, S4, m4, neg, np.float32(1.0))
    assert e6[0, 0] == np.float32(float(g["err6_block1"][0])) and e4[0, 0] == 0
    assert e6[0, 1] == 0 and e4[0, 1] == np.float32(float(g["err4_block2"][0]))


def _four_grid_case(seed, M=8, K=128, j=-5):
    """Blocks x = c·s·2^j with c on the E2M1 grid up to 4 and one |c| = 4."""
    rng = np.random.default_rng(seed)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4])
    nb = K // 16
    c = rng.choice(grid, size=(M, nb, 16)) * rng.choice([-1, 1], size=(M, nb, 16))
    c[:, :, 3] = 4.0 * rng.choice([-1, 1], size=(M, nb))
    s = oracle.e4m3_decode(rng.integers(1, 0x7F, size=(M, nb)))
    x = c * s[:, :, None] * 2.0 ** j
    x[0, 0, :] = 0.0
    x[0, 0, 0] = 2688.0 * 2.0 ** j                          # g = 2^j exactly
    return x.reshape(M, K)


def test_lossless_on_the_four_grid():
    for seed in range(4):
        x = _four_grid_case(seed)
        bits = to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(oracle.bf16_bits_to_f32(bits).astype(np.float64), x)   # bf16-exact
        codes, scales, g = oracle.quantize(bits, adaptive46=True)
        assert np.array_equal(oracle.dequantize(codes, scales, g), x), seed
        # the amax→6 encoding alone is not lossless here (the test is not vacuous)
        c6, s6, g6 = oracle.quantize(bits)
        lossy = (oracle.dequantize(c6, s6, g6) != x).reshape(x.shape[0], -1, 16).any(axis=2)
        assert lossy.mean() > 0.5


def _block_err64(x, codes, scales, g):
    d = oracle.dequantize(codes, scales, g) - x.astype(np.float64)
    return (d * d).reshape(x.shape[0], -1, 16).sum(axis=2)


def test_never_worse_than_six_and_both_targets_used():
    x = random_matrix(7, 64, 512, sigma=1.0, outliers=True)
    xf = oracle.bf16_bits_to_f32(x)
    ca, sa, ga = oracle.quantize(x, adaptive46=True)
    c6, s6, g6 = oracle.quantize(x)
    assert ga == g6
    ea, e6 = _block_err64(xf, ca, sa, ga), _block_err64(xf, c6, s6, g6)
    assert np.all(ea <= e6 * (1 + 1e-5) + 1e-300)
    changed = (sa != s6)
    assert 0.05 < changed.mean() < 0.95, changed.mean()
    assert np.all(ea[changed] < e6[changed] * (1 + 1e-5))


def test_choice_matches_exact_rationals():
    # brute force: exact block errors of both encodings decide the same way,
    # except where they agree to within 1e-5 (binary32 rounding may then tip)
    x = random_matrix(11, 4, 128, sigma=1.0, outliers=False)
    xf = oracle.bf16_bits_to_f32(x)
    ca, sa, ga = oracle.quantize(x, adaptive46=True)
    c6, s6, g = oracle.quantize(x)
    rows, nb = x.shape[0], x.shape[1] // 16
    # the amax→4 encoding, isolated by forcing every block to it through the oracle steps
    S4, m4 = oracle.nvfp4._encode_blocks(np.abs(xf).reshape(rows, nb, 16), g, 4.0)
    sign = np.signbit(xf).reshape(rows, nb, 16)
    u6 = oracle.unpack_nibbles(c6).reshape(rows, nb, 16)
    for i in range(rows):
        for b in range(nb):
            def exact_err(S, mags, negs):
                sv = Fraction(float(oracle.e4m3_decode(np.array([S]))[0])) * Fraction(float(g))
                tot = Fraction(0)
                for k in range(16):
                    v = Fraction(float(oracle.E2M1_VALUES[mags[k]])) * sv
                    v = -v if negs[k] else v
                    d = Fraction(float(xf[i, 16 * b + k])) - v
                    tot += d * d
                return tot
            e6 = exact_err(s6[i, b], u6[i, b] & 7, sign[i, b])
            e4 = exact_err(S4[i, b], m4[i, b], sign[i, b])
            if e6 == e4 or abs(e6 - e4) <= Fraction(1, 10 ** 5) * max(e6, e4):
                continue
            assert (sa[i, b] == S4[i, b]) == (e4 < e6) or S4[i, b] == s6[i, b], (i, b)


def test_invariants():
    x = random_matrix(13, 16, 256, sigma=2.0, outliers=True)
    ca, sa, ga = oracle.quantize(x, adaptive46=True)
    # negation flips only the sign bits
    cn, sn, gn = oracle.quantize(x ^ np.uint16(0x8000), adaptive46=True)
    assert gn == ga and np.array_equal(sn, sa)
    assert np.array_equal(cn, ca ^ np.uint8(0x88))
    # scaling by 2^k scales g only
    xs = to_bf16_bits(oracle.bf16_bits_to_f32(x) * np.float32(2.0 ** 9))
    cs, ss, gs = oracle.quantize(xs, adaptive46=True)
    assert gs == np.float32(ga * np.float32(2.0 ** 9))
    assert np.array_equal(cs, ca) and np.array_equal(ss, sa)
