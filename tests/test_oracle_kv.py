"""Pins for the oracle NVFP4 KV cache.

The byte count is checked against the closed form printed on the pages
(4·T·H·d → 9/8·T·H·d bytes, about 3.6×); an append is checked to equal the
quantiser applied to that chunk viewed as [T·H, d] and written at the right
token offset; the dequant chain is checked against the exact dequant equation
where binary32 makes no rounding (power-of-two tensor scale).
"""

import numpy as np
import pytest

import oracle
from workloads import to_bf16_bits


def _kv(seed, T, H=3, D=64, sigma=1.0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, H, D)).astype(np.float32) * sigma
    v = rng.standard_normal((T, H, D)).astype(np.float32) * sigma * 2
    return to_bf16_bits(k), to_bf16_bits(v)


def test_kv_bytes_closed_form(golden):
    g = golden("kv_bytes.txt")
    bf16_per = float(g["bf16_bytes_per_THd"][0])
    nv_per = float(g["nvfp4_bytes_per_THd_num"][0]) / float(g["nvfp4_bytes_per_THd_den"][0])
    for T, H, D in [(880, 24, 128), (65536, 24, 128), (16, 1, 32)]:
        assert oracle.kv_bytes(T, H, D) == nv_per * T * H * D
        ratio = bf16_per * T * H * D / oracle.kv_bytes(T, H, D)
        assert abs(ratio - float(g["ratio_about"][0])) < float(g["ratio_tolerance"][0])
        assert ratio == 32 / 9
    assert oracle.kv_bytes(880, 24, 128, chunks=3) == 9 * 880 * 24 * 128 // 8 + 24


def test_append_equals_quantize_at_offset():
    H, D = 3, 64
    c = oracle.KVCacheRef(40, H, D)
    k1, v1 = _kv(1, 10, H, D)
    k2, v2 = _kv(2, 7, H, D, sigma=3.0)
    c.append(k1, v1)
    snap = c.k_codes.copy()
    c.append(k2, v2)
    assert np.array_equal(c.k_codes[:10], snap[:10])          # first chunk untouched
    qc, qs, qg = oracle.quantize(k2.reshape(7 * H, D))
    assert np.array_equal(c.k_codes[10:17].reshape(7 * H, -1), qc)
    assert np.array_equal(c.k_scales[10:17].reshape(7 * H, -1), qs)
    vc, vs, vg = oracle.quantize(v2.reshape(7 * H, D))
    assert np.array_equal(c.v_codes[10:17].reshape(7 * H, -1), vc)
    assert c.gscale[1] == (qg, vg)
    assert c.chunk_start == [0, 10, 17] and c.n_tokens == 17
    assert not c.k_codes[17:].any()
    with pytest.raises(ValueError):
        c.append(*_kv(3, 30, H, D))


def test_dequant_exact_for_power_of_two_scale():
    # plant 2688·2^-2 so g = 2^-2 exactly: fl32(E2M1·S·g) is then exact and the
    # bf16 output must equal the nearest-even rounding of the exact dequant value
    H, D, T = 2, 32, 5
    k, v = _kv(4, T, H, D)
    kf = oracle.bf16_bits_to_f32(k).copy()
    kf[0, 0, 0] = 672.0
    vf = oracle.bf16_bits_to_f32(v).copy()
    vf[2, 1, 5] = -672.0
    k, v = to_bf16_bits(kf), to_bf16_bits(vf)
    c = oracle.KVCacheRef(8, H, D)
    c.append(k, v)
    assert c.gscale[0] == (np.float32(0.25), np.float32(0.25))
    ko, vo = c.dequant(0, T)
    qk = oracle.dequantize(*oracle.quantize(k.reshape(T * H, D)))
    qv = oracle.dequantize(*oracle.quantize(v.reshape(T * H, D)))
    assert np.array_equal(ko.reshape(T * H, D), oracle.bf16_rne_from_f64(qk))
    assert np.array_equal(vo.reshape(T * H, D), oracle.bf16_rne_from_f64(qv))


def test_dequant_uses_each_chunks_scale():
    H, D = 2, 32
    c = oracle.KVCacheRef(30, H, D)
    a = _kv(5, 6, H, D, sigma=1.0)
    b = _kv(6, 9, H, D, sigma=40.0)
    c.append(*a)
    c.append(*b)
    ko, vo = c.dequant(3, 12)                # crosses the chunk boundary at 6
    ka, _ = c.dequant(3, 6)
    kb, _ = c.dequant(6, 12)
    assert np.array_equal(ko, np.concatenate([ka, kb]))
    # the reconstructed values track the inputs to NVFP4 accuracy in both chunks
    for (kk, _), lo, hi, part in ((a, 3, 6, ka), (b, 0, 6, kb)):
        x = oracle.bf16_bits_to_f32(kk[lo:hi])
        y = oracle.bf16_bits_to_f32(part)
        assert np.linalg.norm(x - y) / np.linalg.norm(x) < 0.15
    with pytest.raises(ValueError):
        c.dequant(0, 16)


def _hand_example_input(golden):
    """The one-token input of the hand-worked dequant example as bf16 bits [1, 1, 32]."""
    g = golden("kv_dequant_hand_example.txt")
    x = np.zeros(32, np.float32)
    x[0] = oracle.bf16_bits_to_f32(np.array([int(g["amax_bits"][0], 16)], np.uint16))[0]
    m, e = (int(v) for v in g["block_amax"])
    x[16] = np.ldexp(np.float32(m), e)
    m, e = (int(v) for v in g["element"])
    x[17] = np.ldexp(np.float32(m), e)
    x[18] = -x[17]
    return g, to_bf16_bits(x).reshape(1, 1, 32)


def test_dequant_hand_example_non_power_of_two_scale(golden):
    # g = 8738133·2^-34: the binary32 product lands on a bf16 tie, so the
    # two-rounding chain, one rounding from binary64 and the other association
    # of the three factors give different bytes (worked by hand in the fixture)
    g, k = _hand_example_input(golden)
    c = oracle.KVCacheRef(1, 1, 32)
    c.append(k, k)
    gk = np.float32(c.gscale[0][0])
    assert gk.view(np.uint32) == int(g["g_bits"][0], 16)
    assert c.k_scales[0, 0, 1] == int(g["scale_byte"][0], 16)
    codes = oracle.unpack_nibbles(c.k_codes[0, 0])
    assert codes[17] == int(g["code"][0], 16) and codes[18] == int(g["code"][0], 16) | 8
    ko, _ = c.dequant(0, 1)
    assert ko[0, 0, 17] == int(g["expected"][0], 16)
    assert ko[0, 0, 18] == int(g["expected_negative"][0], 16)
    # the readings a mistake could take differ here, so the pin separates them
    exact = oracle.dequantize(c.k_codes[0], c.k_scales[0], gk)[0, 17]          # binary64, exact
    assert oracle.bf16_rne_from_f64(exact) == int(g["one_rounding"][0], 16)
    s = np.float32(oracle.e4m3_decode(c.k_scales[0, 0, 1]))
    alt = np.float32(np.float32(1.5) * np.float32(s * gk))
    assert oracle.bf16_rne_from_f64(np.float64(alt)) == int(g["other_association"][0], 16)
    assert int(g["expected"][0], 16) != int(g["one_rounding"][0], 16)
