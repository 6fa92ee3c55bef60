"""GPU parity of the NVFP4 KV cache: every append's codes, scales and tensor
scales bit-exact against the oracle cache, dequant bit-exact against the
oracle's dequant chain; the full 65536-token workload on every chunk."""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_bits, to_np

pytestmark = pytest.mark.gpu


def _small_kv(seed, T, H, D):
    rng = np.random.default_rng(seed)
    f = rng.uniform(0.5, 4.0, size=H).astype(np.float32)
    k = rng.standard_normal((T, H, D)).astype(np.float32) * f[None, :, None]
    v = rng.standard_normal((T, H, D)).astype(np.float32) * f[::-1][None, :, None] * 3
    return workloads.to_bf16_bits(k), workloads.to_bf16_bits(v)


def _compare_cache(gpu, ref, n):
    assert gpu.n_tokens == ref.n_tokens == n
    for a, b, name in ((gpu.k_codes, ref.k_codes, "k_codes"), (gpu.v_codes, ref.v_codes, "v_codes"),
                       (gpu.k_scales, ref.k_scales, "k_scales"), (gpu.v_scales, ref.v_scales, "v_scales")):
        got = to_np(a)[:n]
        bad = np.argwhere(got != b[:n])
        assert bad.size == 0, (name, bad[:5])
    g = to_np(gpu.gscale)[:gpu.n_chunks]
    assert np.array_equal(g, np.array(ref.gscale, dtype=np.float32).reshape(-1, 2))
    assert list(to_np(gpu.chunk_start)[:gpu.n_chunks + 1]) == ref.chunk_start


@pytest.mark.parametrize("H,D", [(3, 64), (24, 128), (1, 32)])
def test_appends_and_dequant_small(H, D):
    sizes = [5, 1, 17, 8, 3]
    cap = sum(sizes) + 4
    gpu = nv.KVCache(cap, H, D, max_chunks=8)
    ref = oracle.KVCacheRef(cap, H, D)
    n = 0
    for i, T in enumerate(sizes):
        announce(f"kv append H={H} D={D} chunk {i} T={T}")
        k, v = _small_kv(100 * i + H, T, H, D)
        gpu.append(bf16_to_dev(k), bf16_to_dev(v))
        ref.append(k, v)
        n += T
        torch.cuda.synchronize()
        _compare_cache(gpu, ref, n)
    for t0, t1 in ((0, n), (3, 9), (6, 7), (n - 3, n), (4, 4)):
        ko, vo = gpu.dequant(t0, t1)
        torch.cuda.synchronize()
        rk, rv = ref.dequant(t0, t1)
        assert np.array_equal(to_bits(ko), rk), (t0, t1)
        assert np.array_equal(to_bits(vo), rv), (t0, t1)


def test_capacity_errors_leave_cache_unchanged():
    gpu = nv.KVCache(10, 2, 32, max_chunks=2)
    k, v = _small_kv(1, 6, 2, 32)
    gpu.append(bf16_to_dev(k), bf16_to_dev(v))
    with pytest.raises(nv.NVFP4Error) as e:
        gpu.append(bf16_to_dev(k), bf16_to_dev(v))          # 12 > 10 tokens
    assert e.value.status == 3 and gpu.n_tokens == 6 and gpu.n_chunks == 1
    k2, v2 = _small_kv(2, 4, 2, 32)
    gpu.append(bf16_to_dev(k2), bf16_to_dev(v2))
    assert gpu.n_tokens == 10 and gpu.n_chunks == 2


def test_full_workload_every_chunk():
    # the 65536-token workload: 74 appends of 880 tokens and one of 416, every
    # chunk's codes, scales and tensor scales and the whole read-back bit-exact
    K, V, sizes = workloads.kv()
    H, D = workloads.HEADS, workloads.HEAD_DIM
    T = K.shape[0]
    announce(f"kv full workload: {len(sizes)} appends, {T} tokens")
    gpu = nv.KVCache(T, H, D, max_chunks=len(sizes))
    kd, vd = bf16_to_dev(K), bf16_to_dev(V)
    starts = np.r_[0, np.cumsum(sizes)]
    for i, n in enumerate(sizes):
        gpu.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]])
    ko, vo = gpu.dequant(0, T)
    torch.cuda.synchronize()
    del kd, vd
    assert gpu.n_tokens == T and gpu.n_chunks == len(sizes)
    announce("  oracle cache")
    ref = oracle.KVCacheRef(T, H, D)
    for i in range(len(sizes)):
        ref.append(K[starts[i]:starts[i + 1]], V[starts[i]:starts[i + 1]])
    _compare_cache(gpu, ref, T)
    announce("  oracle dequant")
    rk, rv = ref.dequant(0, T)
    assert np.array_equal(to_bits(ko), rk)
    assert np.array_equal(to_bits(vo), rv)
    # storage closed form: 9/8 bytes per element for K and V together
    nbytes = sum(t.numel() for t in (gpu.k_codes, gpu.v_codes, gpu.k_scales, gpu.v_scales))
    assert nbytes * 8 == 9 * T * H * D


@pytest.mark.parametrize("adaptive", [False, True])
def test_eight_frame_chunks(adaptive):
    # the pages' KV chunk of 8 frames (8 x 880 = 7040 tokens) as the append
    # granularity: the 65536-token workload in 9 chunks of 7040 and one of
    # 2176, every byte and the read-back bit-exact, with the adaptive {4, 6}
    # scale selection the pages pair with it
    K, V, _ = workloads.kv()
    H, D = workloads.HEADS, workloads.HEAD_DIM
    T = K.shape[0]
    sizes = workloads.kv_chunk_sizes(T, 8 * workloads.KV_CHUNK)
    announce(f"kv 8-frame chunks: {sizes[:2]}.. ({len(sizes)} appends), adaptive={adaptive}")
    gpu = nv.KVCache(T, H, D, max_chunks=len(sizes))
    kd, vd = bf16_to_dev(K), bf16_to_dev(V)
    starts = np.r_[0, np.cumsum(sizes)]
    for i in range(len(sizes)):
        gpu.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]], adaptive46=adaptive)
    ko, vo = gpu.dequant(0, T)
    torch.cuda.synchronize()
    del kd, vd
    ref = oracle.KVCacheRef(T, H, D)
    for i in range(len(sizes)):
        ref.append(K[starts[i]:starts[i + 1]], V[starts[i]:starts[i + 1]], adaptive46=adaptive)
    _compare_cache(gpu, ref, T)
    rk, rv = ref.dequant(0, T)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)


def test_eight_frame_chunk_lds_resident_expired_wait_strided():
    # An 8-frame chunk (7040 tokens x 24 heads x 128) is larger than the
    # registers of the single-launch K/V kernel hold; it keeps two blocks per
    # thread and tensor in LDS.  K and V are the column slices of fused QKV
    # rows (token stride 3·H·D).  The first append's waits all expire, so its
    # workgroups read the shares they have not heard from in global memory;
    # the second append uses the normal wait on other data.  Every byte is
    # compared with the oracle.
    H, D, T = 24, 128, 7040
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    L.nvfp4_testing_set_quantize_wait(prev)
    gpu = nv.KVCache(2 * T, H, D, max_chunks=2)
    ref = oracle.KVCacheRef(2 * T, H, D)
    try:
        for rep, (seed, sigma) in enumerate([(41, 2.0), (42, 0.25)]):
            rows = workloads.random_matrix(seed, T, 3 * H * D, sigma=sigma, outliers=True)
            announce(f"kv 7040-token LDS-resident append from fused rows, rep {rep}, wait {'0' if rep == 0 else 'default'}")
            dev_rows = bf16_to_dev(rows)
            L.nvfp4_testing_set_quantize_wait(0 if rep == 0 else prev)
            gpu.append(dev_rows[:, H * D:2 * H * D], dev_rows[:, 2 * H * D:])
            torch.cuda.synchronize()
            del dev_rows
            ref.append(np.ascontiguousarray(rows[:, H * D:2 * H * D]).reshape(T, H, D),
                       np.ascontiguousarray(rows[:, 2 * H * D:]).reshape(T, H, D))
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)
    _compare_cache(gpu, ref, 2 * T)


def test_strided_append_from_fused_rows():
    # K and V read in place as column slices of a [T, 3·H·D] row-major matrix
    # (the layout of a fused QKV projection output), token stride 3·H·D
    H, D, T = 24, 128, 300
    rows = workloads.random_matrix(31, T, 3 * H * D, sigma=2.0, outliers=True)
    dev_rows = bf16_to_dev(rows)
    gpu = nv.KVCache(T + 10, H, D, max_chunks=2)
    gpu.append(dev_rows[:, H * D:2 * H * D], dev_rows[:, 2 * H * D:])
    ref = oracle.KVCacheRef(T + 10, H, D)
    ref.append(np.ascontiguousarray(rows[:, H * D:2 * H * D]).reshape(T, H, D),
               np.ascontiguousarray(rows[:, 2 * H * D:]).reshape(T, H, D))
    torch.cuda.synchronize()
    _compare_cache(gpu, ref, T)
    ko, vo = gpu.dequant(0, T)
    rk, rv = ref.dequant(0, T)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)


def test_many_chunks_dequant():
    # more appends than the dequant kernel keeps in LDS (it then searches the
    # chunk starts in global memory)
    H, D, n = 1, 32, 2100
    gpu = nv.KVCache(n, H, D, max_chunks=n)
    ref = oracle.KVCacheRef(n, H, D)
    rng = np.random.default_rng(77)
    kall = workloads.to_bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32) *
                                  rng.uniform(0.1, 10, size=(n, 1, 1)).astype(np.float32))
    vall = workloads.to_bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32))
    kd, vd = bf16_to_dev(kall), bf16_to_dev(vall)
    announce(f"kv {n} one-token appends")
    for t in range(n):
        gpu.append(kd[t:t + 1], vd[t:t + 1])
        ref.append(kall[t:t + 1], vall[t:t + 1])
    ko, vo = gpu.dequant(0, n)
    k2, v2 = gpu.dequant(1234, 1300)
    torch.cuda.synchronize()
    rk, rv = ref.dequant(0, n)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)
    rk2, rv2 = ref.dequant(1234, 1300)
    assert np.array_equal(to_bits(k2), rk2) and np.array_equal(to_bits(v2), rv2)


def test_dequant_hand_example_non_power_of_two_scale(golden):
    # the hand-worked case where fl32(E2M1·S)·g lands on a bf16 tie: the GPU
    # append gives the fixture's g, scale byte and codes, and its dequant the
    # fixture's two-rounding result (not one rounding, not the other association)
    g = golden("kv_dequant_hand_example.txt")
    x = np.zeros(32, np.float32)
    x[0] = oracle.bf16_bits_to_f32(np.array([int(g["amax_bits"][0], 16)], np.uint16))[0]
    m, e = (int(v) for v in g["block_amax"])
    x[16] = np.ldexp(np.float32(m), e)
    m, e = (int(v) for v in g["element"])
    x[17] = np.ldexp(np.float32(m), e)
    x[18] = -x[17]
    k = workloads.to_bf16_bits(x).reshape(1, 1, 32)
    announce("kv dequant hand-worked example")
    kv = nv.KVCache(4, 1, 32, max_chunks=2)
    kv.append(bf16_to_dev(k), bf16_to_dev(k))
    ko, vo = kv.dequant(0, 1)
    torch.cuda.synchronize()
    assert to_np(kv.gscale)[0, 0].view(np.uint32) == int(g["g_bits"][0], 16)
    assert to_np(kv.k_scales)[0, 0, 1] == int(g["scale_byte"][0], 16)
    kb = to_bits(ko)
    assert kb[0, 0, 17] == int(g["expected"][0], 16) and kb[0, 0, 18] == int(g["expected_negative"][0], 16)
    assert np.array_equal(to_bits(vo), kb)
