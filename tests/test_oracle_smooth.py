"""Pins for the K-smoothing oracle (oracle/smooth.py) and the smoothed cache.

* the hand-worked chunk of tests/golden/k_center_hand_example.txt (a bf16 tie
  of the mean, grid ties, saturated keys, a negative mean);
* the centre against an exact rational brute force (Python integers and
  Fractions: the grid rounding, the exact sum, the exact mean rounded once to
  bf16) on random chunks that hold sub-grid values, grid ties and saturated
  keys;
* closed forms: a constant channel is its own centre and smooths to +0; a
  channel shifted by an integer c moves its centre to the rounding of the
  shifted mean; the centre ignores the order of the tokens;
* smoothed keys against the exact difference rounded once to bf16 (the
  binary32 step can never change that rounding: see the test);
* the smoothed cache: an append equals quantising the smoothed keys at the
  right offset, V is untouched, a chunk whose smoothed keys are exact in NVFP4
  reads back exactly, attention over such a cache equals attention over the
  original keys, and smoothing lowers the read-back error of keys whose
  channels carry offsets (its purpose).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import to_bf16_bits


def _bf16_bits_nearest(q: Fraction) -> int:
    """bf16 bits of the value nearest to the rational q (ties to even), by
    exhaustive comparison with the two neighbouring bf16 values."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 7, -133)
    lo = (a // quantum) * quantum
    hi = lo + quantum
    if a - lo < hi - a:
        v = lo
    elif hi - a < a - lo:
        v = hi
    else:
        v = lo if (lo / quantum) % 2 == 0 else hi
    f32 = np.float32(float(v))
    assert Fraction(float(f32)) == v
    return sign | int(f32.view(np.uint32) >> 16)


def _center_fraction(keys_f32: np.ndarray) -> np.ndarray:
    """The centre of every channel of [T, H, D] float32 keys, exactly: each key
    rounded to the 2^-24 grid (Python's round: ties to even), saturated at
    2^38 steps, summed as integers, divided by T as a Fraction, rounded once."""
    T, H, D = keys_f32.shape
    out = np.zeros((H, D), np.uint16)
    for h in range(H):
        for j in range(D):
            s = 0
            for t in range(T):
                z = round(Fraction(float(keys_f32[t, h, j])) * 2 ** 24)
                s += max(-(1 << 38), min(1 << 38, z))
            out[h, j] = _bf16_bits_nearest(Fraction(s, T) / 2 ** 24)
    return out


def _awkward_keys(seed, T, H, D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, H, D)) * rng.uniform(0.01, 30.0, size=(1, H, D)) + \
        rng.standard_normal((1, H, D)) * 5
    kind = rng.integers(0, 6, size=k.shape)
    k = np.where(kind == 0, rng.integers(-7, 8, size=k.shape) * 2.0 ** -25, k)    # grid ties, sub-grid
    k = np.where(kind == 1, rng.integers(-3, 4, size=k.shape) * 2.0 ** -27, k)    # below half a step
    k = np.where(kind == 2, np.sign(rng.standard_normal(k.shape)) * rng.uniform(9000, 70000, k.shape), k)
    return to_bf16_bits(k.astype(np.float32))


def test_center_hand_example(golden):
    g = golden("k_center_hand_example.txt")
    T = int(g["T"][0])
    k = np.zeros((T, 1, 32), np.uint16)
    for c in range(4):
        k[:, 0, c] = [int(v, 16) for v in g[f"ch{c}_keys"]]
    mu = oracle.k_center(k)
    assert mu[0, :4].tolist() == [int(v, 16) for v in g["centres"]]
    assert not mu[0, 4:].any()
    sk = oracle.smooth_keys(k, mu)
    assert sk[:, 0, 0].tolist() == [int(v, 16) for v in g["smoothed_ch0"]]
    assert sk[:, 0, 2].tolist() == [int(v, 16) for v in g["smoothed_ch2"]]


@pytest.mark.parametrize("seed,T", [(1, 1), (2, 2), (3, 3), (4, 7), (5, 17), (6, 40)])
def test_center_exact_brute_force(seed, T):
    k = _awkward_keys(seed, T, 2, 32)
    kf = oracle.bf16_bits_to_f32(k)
    assert np.array_equal(oracle.k_center(k), _center_fraction(kf))


def test_constant_channel_and_permutation():
    rng = np.random.default_rng(8)
    k = to_bf16_bits((rng.standard_normal((9, 2, 32)) * 4).astype(np.float32))
    c = to_bf16_bits(np.float32([3.75, -1024.0, 2.0 ** -17, 0.0]))
    for i, cv in enumerate(c):
        k[:, i % 2, 5 + i] = cv                    # constant channels
    mu = oracle.k_center(k)
    for i, cv in enumerate(c):
        assert mu[i % 2, 5 + i] == cv
    sk = oracle.smooth_keys(k, mu)
    for i in range(len(c)):
        assert not sk[:, i % 2, 5 + i].any()       # +0 exactly
    perm = rng.permutation(9)
    assert np.array_equal(oracle.k_center(k[perm]), mu)


def test_integer_shift_moves_the_centre():
    # integer keys (exact on the grid, no saturation): the centre of K + c is
    # the once-rounded exact mean of K + c, c an integer per channel
    rng = np.random.default_rng(9)
    base = rng.integers(-20, 21, size=(11, 1, 32)).astype(np.float32)
    shift = (rng.integers(-6, 7, size=(1, 1, 32)) * 16).astype(np.float32)
    k = to_bf16_bits(base + shift)
    assert np.array_equal(oracle.bf16_bits_to_f32(k), base + shift)      # exact in bf16
    mu = oracle.k_center(k)
    for j in range(32):
        exact = Fraction(int((base[:, 0, j] + shift[0, 0, j]).sum()), 11)
        assert mu[0, j] == _bf16_bits_nearest(exact)


def test_smoothed_keys_single_rounding():
    # K and the centre are bf16: their exact difference needs more than 24
    # bits only when the centre is below 2^-16 of K, and then the difference
    # lies within 2^-16 of K, far from any bf16 tie — so fl32 then bf16 is the
    # single nearest-even rounding of the exact difference
    k = _awkward_keys(10, 13, 2, 32)
    rng = np.random.default_rng(11)
    mu = to_bf16_bits((rng.standard_normal((2, 32)) * rng.choice([1e-9, 1e-3, 1.0, 300.0], (2, 32))).astype(np.float32))
    sk = oracle.smooth_keys(k, mu)
    kf, mf = oracle.bf16_bits_to_f32(k), oracle.bf16_bits_to_f32(mu)
    for t in range(13):
        for h in range(2):
            for j in range(32):
                d = Fraction(float(kf[t, h, j])) - Fraction(float(mf[h, j]))
                assert sk[t, h, j] == _bf16_bits_nearest(d), (t, h, j)
    zero = np.zeros((2, 32), np.uint16)
    k2 = k.copy()
    k2[0, 0, 0] = 0x8000                           # -0 stays -0 under a zero centre
    assert np.array_equal(oracle.smooth_keys(k2, zero), k2)


def test_smoothed_append_is_quantize_of_smoothed_keys():
    H, D = 3, 64
    rng = np.random.default_rng(12)
    k1 = to_bf16_bits((rng.standard_normal((10, H, D)) + 7).astype(np.float32))
    v1 = to_bf16_bits(rng.standard_normal((10, H, D)).astype(np.float32))
    k2 = to_bf16_bits((rng.standard_normal((6, H, D)) * 3 - 20).astype(np.float32))
    v2 = to_bf16_bits(rng.standard_normal((6, H, D)).astype(np.float32))
    c = oracle.KVCacheRef(20, H, D, smooth_k=True)
    plain = oracle.KVCacheRef(20, H, D)
    for k, v in ((k1, v1), (k2, v2)):
        c.append(k, v, adaptive46=True)
        plain.append(k, v, adaptive46=True)
    mu2 = oracle.k_center(k2)
    qc, qs, qg = oracle.quantize(oracle.smooth_keys(k2, mu2).reshape(6 * H, D), adaptive46=True)
    assert np.array_equal(c.k_codes[10:16].reshape(6 * H, -1), qc)
    assert np.array_equal(c.k_scales[10:16].reshape(6 * H, -1), qs)
    assert c.gscale[1][0] == qg and np.array_equal(c.k_center[1], mu2)
    assert np.array_equal(c.v_codes, plain.v_codes) and np.array_equal(c.v_scales, plain.v_scales)
    assert [g[1] for g in c.gscale] == [g[1] for g in plain.gscale]
    _, vd = c.dequant(0, 16)
    _, vp = plain.dequant(0, 16)
    assert np.array_equal(vd, vp)


def _lossless_smoothed_chunk(seed, T, H, D):
    """Keys = per-channel offsets (multiples of 8) + E2M1 values, the second
    half of the tokens holding the negated values of the first (each
    channel's mean is its offset): the smoothed keys are the E2M1 values,
    every 16-block holds ±6, and one block of head 0 holds 112 times E2M1
    values with 672 = 2688·2^-2 among them, which makes g = 2^-2; so NVFP4
    holds the smoothed keys exactly."""
    rng = np.random.default_rng(seed)
    grid = np.array([0.5, 1, 1.5, 2, 3, 4, 6])
    q = rng.choice(grid, size=(T // 2, H, D)) * rng.choice([-1, 1], size=(T // 2, H, D))
    q[:, :, ::16] = 6.0
    q[0, 0, :16] *= 112.0
    q = np.concatenate([q, -q])
    off = (rng.integers(-8, 9, size=(1, H, D)) * 8).astype(np.float64)
    k = (q + off).astype(np.float32)
    assert np.array_equal(oracle.bf16_bits_to_f32(to_bf16_bits(k)), k)
    return to_bf16_bits(k), off


def test_lossless_chunk_reads_back_exactly():
    H, D, T = 2, 32, 8
    k, off = _lossless_smoothed_chunk(13, T, H, D)
    c = oracle.KVCacheRef(T, H, D, smooth_k=True)
    c.append(k, k)
    assert np.array_equal(oracle.bf16_bits_to_f32(c.k_center[0]), off[0].astype(np.float32))
    assert c.gscale[0][0] == np.float32(0.25)
    kd, _ = c.dequant(0, T)
    assert np.array_equal(kd, k)
    kv, _ = c.values(np.arange(T))
    assert np.array_equal(kv, oracle.bf16_bits_to_f32(k).astype(np.float64))


def test_attention_over_smoothed_cache_sees_the_keys():
    H, D, T = 2, 32, 8
    k, _ = _lossless_smoothed_chunk(14, T, H, D)
    rng = np.random.default_rng(15)
    v = to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32))
    q = to_bf16_bits((rng.standard_normal((5, H, D)) * 0.01).astype(np.float32))
    c = oracle.KVCacheRef(T, H, D, smooth_k=True)
    c.append(k, v)
    o, _ = oracle.kv_attention_ref(q, c, [(0, T)])
    _, vv = c.values(np.arange(T))
    ref = oracle.attention_ref(oracle.bf16_bits_to_f32(q), oracle.bf16_bits_to_f32(k), vv)
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def test_smoothing_lowers_the_error_of_offset_channels():
    # keys whose channels carry offsets much larger than their spread: the
    # offsets set every block scale of an unsmoothed chunk, so the spread is
    # lost; the smoothed chunk quantises the spread alone
    rng = np.random.default_rng(16)
    T, H, D = 64, 4, 64
    k = rng.standard_normal((T, H, D)) + rng.standard_normal((1, H, D)) * 20
    kb = to_bf16_bits(k.astype(np.float32))
    kf = oracle.bf16_bits_to_f32(kb).astype(np.float64)
    errs = []
    for smooth in (False, True):
        c = oracle.KVCacheRef(T, H, D, smooth_k=smooth)
        c.append(kb, kb)
        kv, _ = c.values(np.arange(T))
        errs.append(np.sqrt(np.mean((kv - kf) ** 2)))
    assert errs[1] < 0.25 * errs[0], errs
