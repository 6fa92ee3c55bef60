"""Pins for the attention oracle (oracle/attention.py).

attention_ref is the textbook operator; it is pinned by closed forms (zero
queries give the mean of V, a single key gives its V row, V scaled by 2 gives
O scaled by 2), by key-permutation invariance, and by torch's
scaled_dot_product_attention in float64 (a library routine).  kv_attention_ref
is pinned by caches that hold K and V losslessly: then it must equal
attention_ref on the original values bit for bit, across appends with
different tensor scales and for a list of token ranges.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import to_bf16_bits


def _rand(seed, Tq, Tk, H, D, sk=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Tq, H, D)), sk * rng.standard_normal((Tk, H, D)),
            rng.standard_normal((Tk, H, D)))


def test_zero_queries_give_the_mean_of_v():
    q, k, v = _rand(1, 3, 17, 2, 32)
    o = oracle.attention_ref(np.zeros_like(q), k, v)
    for i in range(3):
        np.testing.assert_allclose(o[i], v.mean(axis=0), rtol=1e-14, atol=1e-15)


def test_single_key_gives_its_value():
    q, k, v = _rand(2, 5, 1, 3, 32)
    o = oracle.attention_ref(q, k, v)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))


def test_value_scaling_and_key_permutation():
    q, k, v = _rand(3, 6, 40, 2, 64)
    o = oracle.attention_ref(q, k, v)
    assert np.array_equal(oracle.attention_ref(q, k, 2 * v), 2 * o)
    perm = np.random.default_rng(3).permutation(40)
    np.testing.assert_allclose(oracle.attention_ref(q, k[perm], v[perm]), o, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("Tq,Tk,H,D,scale", [(7, 33, 2, 32, None), (16, 300, 3, 128, None), (5, 9, 1, 64, 0.37)])
def test_matches_torch_sdpa_float64(Tq, Tk, H, D, scale):
    q, k, v = _rand(4 + Tk, Tq, Tk, H, D, sk=2.0)
    o = oracle.attention_ref(q, k, v, scale)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))     # [H, T, D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    np.testing.assert_allclose(o, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-13)


def _lossless_kv(seed, T, H, D, j):
    """K or V values c·s·2^j that NVFP4 holds exactly: every 16-block has a
    largest |c| of 6 and a scale byte in 0x30..0x40 (0.5..2), except the first
    block of token 0, head 0, whose scale is 448 (byte 0x7E) with c = 6 first,
    so the tensor amax 6·448·2^j gives g = 2^j exactly."""
    rng = np.random.default_rng(seed)
    e2 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    nb = D // 16
    c = rng.choice(e2, size=(T, H, nb, 16)) * rng.choice([-1, 1], size=(T, H, nb, 16))
    c[..., 0] = 6.0 * rng.choice([-1, 1], size=(T, H, nb))
    c[0, 0, 0, 0] = 6.0
    sb = rng.integers(0x30, 0x41, size=(T, H, nb))
    sb[0, 0, 0] = 0x7E
    s = oracle.e4m3_decode(sb)
    return (c * s[..., None] * 2.0 ** j).reshape(T, H, D)


def test_cache_attention_equals_plain_attention_on_lossless_values():
    # two appends, K and V with their own tensor scales (2^-4, 2^-3), then
    # (2^-1, 2^-6); the queries are zero on the
    # first 16 coordinates (the block that holds the amax) so the scores stay
    # moderate
    H, D = 2, 32
    parts = [(_lossless_kv(10, 6, H, D, -4), _lossless_kv(11, 6, H, D, -3)),
             (_lossless_kv(12, 9, H, D, -1), _lossless_kv(13, 9, H, D, -6))]
    cache = oracle.KVCacheRef(15, H, D)
    for k, v in parts:
        kb, vb = to_bf16_bits(k.astype(np.float32)), to_bf16_bits(v.astype(np.float32))
        assert np.array_equal(oracle.bf16_bits_to_f32(kb), k) and np.array_equal(oracle.bf16_bits_to_f32(vb), v)
        cache.append(kb, vb)
    assert cache.gscale == [(np.float32(2.0 ** -4), np.float32(2.0 ** -3)),
                            (np.float32(2.0 ** -1), np.float32(2.0 ** -6))]
    kall = np.concatenate([p[0] for p in parts])
    vall = np.concatenate([p[1] for p in parts])
    rng = np.random.default_rng(14)
    q = to_bf16_bits(rng.standard_normal((4, H, D)).astype(np.float32))
    qf = oracle.bf16_bits_to_f32(q).astype(np.float64)
    qf_masked = qf.copy()
    qf_masked[:, :, :16] = 0.0
    q = to_bf16_bits(qf_masked.astype(np.float32))
    o64, obits = oracle.kv_attention_ref(q, cache, [(0, 15)])
    assert np.array_equal(o64, oracle.attention_ref(qf_masked, kall, vall))
    assert np.array_equal(obits, oracle.bf16_rne_from_f64(o64))
    # a list of disjoint ranges is the attention over the concatenated tokens
    ranges = [(0, 2), (4, 7), (12, 15)]
    t = oracle.range_tokens(ranges)
    assert list(t) == [0, 1, 4, 5, 6, 12, 13, 14]
    o2, _ = oracle.kv_attention_ref(q, cache, ranges)
    assert np.array_equal(o2, oracle.attention_ref(qf_masked, kall[t], vall[t]))
    with pytest.raises(ValueError):
        oracle.range_tokens([(0, 4), (3, 6)])
