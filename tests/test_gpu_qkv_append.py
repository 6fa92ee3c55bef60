"""GPU tests of nvfp4_qkv_append: the QKV projection with its K and V
appended to the NVFP4 cache from the GEMM's tile maxima.

* Against the unfused path on the same device (nvfp4_linear, then
  nvfp4_kv_append_ex on the K and V column slices of its output): the QKV
  output and every cache byte (codes, scales, tensor scales, chunk starts) are
  identical, over a sequence of appends of ragged sizes, with and without the
  adaptive {4, 6} scales, on the fused path and on the fallback (a K/V slice
  width that the GEMM tile does not divide).
* Against the oracle (bf16 QKV from oracle.gemm_ref, then KVCacheRef.append of
  its K and V slices): the QKV output within the GEMM tolerance, equal tensor
  scales, equal bytes in every 16-element block whose GPU QKV values are
  bit-identical to the oracle's, and at least 99.9 % equal bytes overall (the
  fp32 accumulation order can flip a last bf16 bit of an output; the same
  reading as the FFN hand-off).
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import GEMM_TOL, announce, bf16_to_dev, gemm_errors, to_bits, to_np

pytestmark = pytest.mark.gpu


def _weights(seed, heads, head_dim, D):
    rng = np.random.default_rng(seed)
    N = 3 * heads * head_dim
    w = workloads.to_bf16_bits((rng.standard_normal((N, D)) * 0.02).astype(np.float32))
    b = workloads.to_bf16_bits((rng.standard_normal(N) * 0.01).astype(np.float32))
    return w, b


def _frames(seed, sizes, D):
    rng = np.random.default_rng(seed)
    out = []
    for i, T in enumerate(sizes):
        x = rng.standard_normal((T, D)).astype(np.float32) * np.float32(1 + i % 3)
        out.append(workloads.to_bf16_bits(x))
    return out


def _cache_state(c):
    return [to_np(t) for t in (c.k_codes, c.k_scales, c.v_codes, c.v_scales, c.gscale, c.chunk_start)]


@pytest.mark.parametrize("heads,head_dim,D,sizes,adaptive", [
    (24, 128, 3072, [880, 100, 1, 300], False),     # the DiT's 24 heads of 128: fused path
    (24, 128, 3072, [880, 257], True),              # adaptive {4, 6} scales for the appends
    (3, 32, 256, [64, 33, 7], False),               # K/V slices 96 wide: the unfused fallback
])
def test_qkv_append_equals_linear_then_append(heads, head_dim, D, sizes, adaptive):
    announce(f"qkv_append heads={heads} head_dim={head_dim} D={D} sizes={sizes} adaptive={adaptive}")
    hd = heads * head_dim
    w, b = _weights(3, heads, head_dim, D)
    wq, ws_, wg = nv.quantize(bf16_to_dev(w))
    bias = bf16_to_dev(b)
    cap = sum(sizes)
    fused = nv.KVCache(cap, heads, head_dim, max_chunks=len(sizes))
    plain = nv.KVCache(cap, heads, head_dim, max_chunks=len(sizes))
    for x in _frames(4, sizes, D):
        xd = bf16_to_dev(x)
        q1 = fused.qkv_append(xd, wq, ws_, wg, bias=bias, adaptive46=adaptive)
        q2 = nv.linear(xd, wq, ws_, wg, bias=bias)
        plain.append(q2[:, hd:2 * hd], q2[:, 2 * hd:], adaptive46=adaptive)
        torch.cuda.synchronize()
        assert torch.equal(q1, q2)
    assert fused.n_tokens == plain.n_tokens == cap and fused.n_chunks == len(sizes)
    for a, b_, name in zip(_cache_state(fused), _cache_state(plain),
                           ("k_codes", "k_scales", "v_codes", "v_scales", "gscale", "chunk_start")):
        assert np.array_equal(a, b_), name


def test_qkv_append_against_oracle():
    heads, head_dim, D, T = 24, 128, 3072, 880
    hd = heads * head_dim
    announce(f"qkv_append against the oracle, T={T}")
    w, b = _weights(5, heads, head_dim, D)
    (x,) = _frames(6, [T], D)
    wq, ws_, wg = nv.quantize(bf16_to_dev(w))
    cache = nv.KVCache(T, heads, head_dim, max_chunks=1)
    qkv = cache.qkv_append(bf16_to_dev(x), wq, ws_, wg, bias=bf16_to_dev(b))
    torch.cuda.synchronize()
    c64, cref = oracle.gemm_ref(*oracle.quantize(x), *oracle.quantize(w), bias_bits=b)
    got = to_bits(qkv)
    e_ref, e64 = gemm_errors(got, c64, cref)
    assert e_ref <= GEMM_TOL and e64 <= GEMM_TOL, (e_ref, e64)
    ref = oracle.KVCacheRef(T, heads, head_dim)
    ref.append(np.ascontiguousarray(cref[:, hd:2 * hd]).reshape(T, heads, head_dim),
               np.ascontiguousarray(cref[:, 2 * hd:]).reshape(T, heads, head_dim))
    assert np.array_equal(to_np(cache.gscale)[0], np.array(ref.gscale[0], dtype=np.float32))
    for i, (lo, name) in enumerate(((hd, "K"), (2 * hd, "V"))):
        same = (got[:, lo:lo + hd] == cref[:, lo:lo + hd]).reshape(T, hd // 16, 16).all(axis=2)
        codes = to_np(cache.k_codes if i == 0 else cache.v_codes).reshape(T, hd // 16, 8)
        scales = to_np(cache.k_scales if i == 0 else cache.v_scales).reshape(T, hd // 16)
        rc = (ref.k_codes if i == 0 else ref.v_codes).reshape(T, hd // 16, 8)
        rs = (ref.k_scales if i == 0 else ref.v_scales).reshape(T, hd // 16)
        assert np.array_equal(codes[same], rc[same]) and np.array_equal(scales[same], rs[same]), name
        eq = (codes == rc).all(axis=2) & (scales == rs)
        announce(f"  {name}: {same.mean():.5f} of blocks bit-identical in QKV, {eq.mean():.5f} equal bytes")
        assert eq.mean() >= 0.999, name
