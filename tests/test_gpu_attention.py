"""GPU parity of the attention over the NVFP4 KV cache (nvfp4_kv_attention)
and of its bf16-K/V twin (nvfp4_attention_bf16), against the binary64 oracle
(oracle/attention.py).

Tolerance: the GPU path rounds two quantities to bf16, the probabilities
times g_V before the P·V product and the output; everything else is exact
(the dequantised K and V, Q in fp16, their products) or fp32.  Each bf16
rounding is at most 2^-9 relative, so the output is checked against the
binary64 oracle within ATTN_TOL = 2·2^-9 normwise, per head.  The oracle's
own bf16 rounding of that result is another 2^-9 away from it, so against the
bf16-rounded oracle the bound is ATTN_TOL_BF16 = 3·2^-9 (a single key, where
nothing averages out, reaches it).
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_bits

pytestmark = pytest.mark.gpu

ATTN_TOL = 2 * 2.0 ** -9
ATTN_TOL_BF16 = 3 * 2.0 ** -9
D = 128


def _kv_appends(seed, sizes, H):
    rng = np.random.default_rng(seed)
    fk = rng.uniform(0.5, 4.0, size=H).astype(np.float32)
    fv = rng.uniform(0.5, 4.0, size=H).astype(np.float32)
    out = []
    for i, T in enumerate(sizes):
        s = np.float32(1.0 + 2.0 * (i % 3))                # appends with different amax
        k = rng.standard_normal((T, H, D)).astype(np.float32) * fk[None, :, None] * s
        v = rng.standard_normal((T, H, D)).astype(np.float32) * fv[None, :, None] / s
        out.append((workloads.to_bf16_bits(k), workloads.to_bf16_bits(v)))
    return out


def _caches(seed, sizes, H):
    cap = sum(sizes)
    gpu = nv.KVCache(cap, H, D, max_chunks=len(sizes))
    ref = oracle.KVCacheRef(cap, H, D)
    for k, v in _kv_appends(seed, sizes, H):
        gpu.append(bf16_to_dev(k), bf16_to_dev(v))
        ref.append(k, v)
    return gpu, ref


def _queries(seed, Tq, H, sigma=1.0):
    rng = np.random.default_rng(seed)
    return workloads.to_bf16_bits(sigma * rng.standard_normal((Tq, H, D)).astype(np.float32))


def _check(o_bits, o64, o_ref_bits, label):
    got = oracle.bf16_bits_to_f32(o_bits).astype(np.float64)
    ref = oracle.bf16_bits_to_f32(o_ref_bits).astype(np.float64)
    for h in range(o64.shape[1]):
        e64 = np.linalg.norm(got[:, h] - o64[:, h]) / np.linalg.norm(o64[:, h])
        eref = np.linalg.norm(got[:, h] - ref[:, h]) / np.linalg.norm(ref[:, h])
        announce(f"  {label} head {h}: {e64:.3e} vs fp64, {eref:.3e} vs bf16 oracle")
        assert e64 <= ATTN_TOL and eref <= ATTN_TOL_BF16, (label, h, e64, eref)


@pytest.mark.parametrize("sizes,Tq,ranges", [
    ([40, 70, 33], 50, [(0, 143)]),                              # one split, a ragged key tile
    ([40, 70, 33], 129, [(0, 10), (40, 90), (120, 143)]),       # three ranges, ragged query tile
    ([64, 64], 1, [(5, 6)]),                                     # one query, one key
    ([880, 880, 880, 880, 880, 416], 200, [(0, 880), (2640, 4816)]),   # sink + window, several splits
])
def test_kv_attention_against_oracle(sizes, Tq, ranges):
    H = 3
    announce(f"kv attention sizes={sizes} Tq={Tq} ranges={ranges}")
    gpu, ref = _caches(7, sizes, H)
    q = _queries(8, Tq, H)
    o = gpu.attention(bf16_to_dev(q), ranges)
    torch.cuda.synchronize()
    o64, obits = oracle.kv_attention_ref(q, ref, ranges)
    _check(to_bits(o), o64, obits, "nvfp4")


def test_kv_attention_scale_and_strided_queries():
    # Q and O as column slices of wider rows (a fused QKV output), explicit scale
    H, Tq = 2, 70
    gpu, ref = _caches(9, [100, 60], H)
    rows = workloads.random_matrix(10, Tq, 3 * H * D, sigma=1.0)
    qd = bf16_to_dev(rows)[:, :H * D]
    out_rows = torch.zeros((Tq, 2 * H * D), dtype=torch.bfloat16, device="cuda")
    gpu.attention(qd, [(0, 160)], scale=0.05, out=out_rows[:, H * D:])
    torch.cuda.synchronize()
    q = np.ascontiguousarray(rows[:, :H * D]).reshape(Tq, H, D)
    o64, obits = oracle.kv_attention_ref(q, ref, [(0, 160)], scale=0.05)
    got = to_bits(out_rows)
    assert not got[:, :H * D].any()                              # nothing outside the slice
    _check(np.ascontiguousarray(got[:, H * D:]).reshape(Tq, H, D), o64, obits, "strided")


def test_bf16_twin_against_oracle():
    H, Tq, Tk = 2, 150, 3000
    announce(f"bf16 attention twin Tq={Tq} Tk={Tk}")
    rng = np.random.default_rng(11)
    k = workloads.to_bf16_bits(rng.standard_normal((Tk, H, D)).astype(np.float32))
    v = workloads.to_bf16_bits(3 * rng.standard_normal((Tk, H, D)).astype(np.float32))
    q = _queries(12, Tq, H)
    o = nv.attention_bf16(bf16_to_dev(q), bf16_to_dev(k), bf16_to_dev(v))
    torch.cuda.synchronize()
    f = lambda b: oracle.bf16_bits_to_f32(b).astype(np.float64)
    o64 = oracle.attention_ref(f(q), f(k), f(v))
    _check(to_bits(o), o64, oracle.bf16_rne_from_f64(o64), "bf16 twin")


def test_kv_attention_full_cache_sampled_queries():
    # the 65536-token workload (74 appends of 880 + one of 416, 24 heads), one
    # 880-token query chunk over the whole cache, checked on sampled queries
    K, V, sizes = workloads.kv()
    H = workloads.HEADS
    T = K.shape[0]
    gpu = nv.KVCache(T, H, D, max_chunks=len(sizes))
    ref = oracle.KVCacheRef(T, H, D)
    kd, vd = bf16_to_dev(K), bf16_to_dev(V)
    starts = np.r_[0, np.cumsum(sizes)]
    for i in range(len(sizes)):
        gpu.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])
        ref.append(K[starts[i]:starts[i + 1]], V[starts[i]:starts[i + 1]])
    del kd, vd
    q = _queries(13, 880, H)
    announce("kv attention: 880 queries over 65536 tokens x 24 heads")
    o = gpu.attention(bf16_to_dev(q), [(0, T)])
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0:4, np.random.default_rng(13).integers(0, 880, 8), 876:880])
    o64, obits = oracle.kv_attention_ref(q[rows], ref, [(0, T)])
    _check(to_bits(o)[rows], o64, obits, "full cache")


def test_rejects_bad_ranges_and_head_dim():
    gpu, _ = _caches(14, [16], 1)
    q = bf16_to_dev(_queries(15, 4, 1))
    for bad in ([(0, 17)], [(3, 3)], [(0, 8), (4, 12)], [(0, 1)] * 5):
        with pytest.raises(nv.NVFP4Error) as e:
            gpu.attention(q, bad)
        assert e.value.status == 1
    small = nv.KVCache(8, 1, 64, max_chunks=1)
    with pytest.raises((nv.NVFP4Error, ValueError)):
        small.attention(torch.zeros((2, 1, 64), dtype=torch.bfloat16, device="cuda"), [(0, 1)])
