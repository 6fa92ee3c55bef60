"""GPU parity of the K-smoothed NVFP4 KV cache against the oracle
(oracle/smooth.py, KVCacheRef(smooth_k=True)).

* every append's channel centres, codes, scales, tensor scales and chunk
  starts bit-exact, and the read-back (centre added back) bit-exact, over
  ragged appends (1 token included), keys with channel offsets, grid ties,
  sub-grid and saturated keys, with and without the adaptive {4, 6} scales;
* the pages' configuration at full size: 65536 tokens in 8-frame chunks of
  7040 tokens, K-smoothing and adaptive scales, every chunk and the whole
  read-back bit-exact;
* single appends at the boundaries of the single launch's register and LDS
  capacity for a K/V pair (one or both LDS blocks per thread in use, and just
  past them, where the two-pass kernels take over);
* keys read in place as the K slice of a fused QKV output, and
  nvfp4_qkv_append on a smoothed cache equal to nvfp4_linear followed by the
  smoothed append;
* attention over a smoothed cache against the binary64 oracle over the same
  cache (keys E2M1·S·g + μ), within the tolerance of the unsmoothed
  attention: tiles inside one append and tiles spanning several, several
  ranges, several splits;
* the K-smoothing part of the workspace needs no initialisation (appends
  through a workspace whose smoothing part holds garbage are exact).
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_bits, to_np

pytestmark = pytest.mark.gpu

ATTN_TOL = 2 * 2.0 ** -9
ATTN_TOL_BF16 = 3 * 2.0 ** -9


def _offset_keys(seed, T, H, D, awkward=False):
    rng = np.random.default_rng(seed)
    f = rng.uniform(0.5, 4.0, size=(1, H, 1))
    k = rng.standard_normal((T, H, D)) * f + rng.standard_normal((1, H, D)) * 4 * f
    if awkward:
        kind = rng.integers(0, 8, size=k.shape)
        k = np.where(kind == 0, rng.integers(-7, 8, size=k.shape) * 2.0 ** -25, k)     # grid ties, sub-grid
        k = np.where(kind == 1, np.sign(rng.standard_normal(k.shape)) * rng.uniform(9000, 70000, k.shape), k)
    v = rng.standard_normal((T, H, D)) * f[:, ::-1]
    return workloads.to_bf16_bits(k.astype(np.float32)), workloads.to_bf16_bits(v.astype(np.float32))


def _compare(gpu, ref, n):
    assert gpu.n_tokens == ref.n_tokens == n
    for a, b, name in ((gpu.k_codes, ref.k_codes, "k_codes"), (gpu.v_codes, ref.v_codes, "v_codes"),
                       (gpu.k_scales, ref.k_scales, "k_scales"), (gpu.v_scales, ref.v_scales, "v_scales")):
        bad = np.argwhere(to_np(a)[:n] != b[:n])
        assert bad.size == 0, (name, bad[:5])
    nc = gpu.n_chunks
    assert np.array_equal(to_np(gpu.gscale)[:nc], np.array(ref.gscale, dtype=np.float32).reshape(-1, 2))
    assert list(to_np(gpu.chunk_start)[:nc + 1]) == ref.chunk_start
    assert np.array_equal(to_bits(gpu.k_center)[:nc], np.stack(ref.k_center)), "centres"


def _dirty_smoothing_scratch(cache, T):
    """The cache's append workspace for T tokens with its K-smoothing part
    (after the quantiser's own part) filled with garbage: that part needs no
    initialisation."""
    import ctypes as C
    n = C.c_size_t()
    nv.lib().nvfp4_kv_append_workspace(T, cache.desc.heads, cache.desc.head_dim, C.byref(n))
    ws = nv.workspace(cache.workspace_bytes(T), cache.device)
    ws[n.value:].fill_(0xA5)
    return ws


@pytest.mark.parametrize("H,D,adaptive,awkward", [(3, 64, False, False), (24, 128, True, False),
                                                  (2, 32, False, True), (5, 128, True, True)])
def test_smoothed_appends_and_dequant(H, D, adaptive, awkward):
    sizes = [5, 1, 17, 8, 3, 130, 2]
    cap = sum(sizes) + 3
    gpu = nv.KVCache(cap, H, D, max_chunks=8, smooth_k=True)
    ref = oracle.KVCacheRef(cap, H, D, smooth_k=True)
    n = 0
    for i, T in enumerate(sizes):
        announce(f"smoothed append H={H} D={D} adaptive={adaptive} awkward={awkward} chunk {i} T={T}")
        k, v = _offset_keys(100 * i + H, T, H, D, awkward)
        ws = _dirty_smoothing_scratch(gpu, T) if i % 2 else None
        gpu.append(bf16_to_dev(k), bf16_to_dev(v), ws=ws, adaptive46=adaptive)
        ref.append(k, v, adaptive46=adaptive)
        n += T
        torch.cuda.synchronize()
        _compare(gpu, ref, n)
    for t0, t1 in ((0, n), (3, 9), (6, 7), (n - 3, n), (4, 4), (20, 160)):
        ko, vo = gpu.dequant(t0, t1)
        torch.cuda.synchronize()
        rk, rv = ref.dequant(t0, t1)
        assert np.array_equal(to_bits(ko), rk), (t0, t1)
        assert np.array_equal(to_bits(vo), rv), (t0, t1)


def test_eight_frame_chunks_smoothed_adaptive_full_size():
    # the pages' KV configuration: chunks of 8 frames (7040 tokens), K-smoothing
    # and adaptive {4, 6} scales, over the 65536-token workload
    K, V, _ = workloads.kv()
    H, D = workloads.HEADS, workloads.HEAD_DIM
    T = K.shape[0]
    sizes = workloads.kv_chunk_sizes(T, 8 * workloads.KV_CHUNK)
    announce(f"smoothed 8-frame chunks: {len(sizes)} appends of {sizes[0]}.., {T} tokens")
    gpu = nv.KVCache(T, H, D, max_chunks=len(sizes), smooth_k=True)
    kd, vd = bf16_to_dev(K), bf16_to_dev(V)
    starts = np.r_[0, np.cumsum(sizes)]
    for i in range(len(sizes)):
        gpu.append(kd[starts[i]:starts[i + 1]], vd[starts[i]:starts[i + 1]], adaptive46=True)
    ko, vo = gpu.dequant(0, T)
    torch.cuda.synchronize()
    del kd, vd
    announce("  oracle cache")
    ref = oracle.KVCacheRef(T, H, D, smooth_k=True)
    for i in range(len(sizes)):
        ref.append(K[starts[i]:starts[i + 1]], V[starts[i]:starts[i + 1]], adaptive46=True)
    _compare(gpu, ref, T)
    rk, rv = ref.dequant(0, T)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)


@pytest.mark.parametrize("T,smooth,adaptive", [(6000, True, False), (8192, True, True), (8192, False, False),
                                                (8200, True, False)])
def test_pair_register_and_lds_capacity_boundaries(T, smooth, adaptive):
    # A K/V append of 24 heads x 128 past the registers of the single launch:
    # 6000 tokens use one of the two LDS blocks per thread and tensor, 8192
    # fill both exactly, 8200 go to the two-pass kernels.  Keys with channel
    # offsets, with and without K-smoothing; every byte, the centres and the
    # read-back bit-exact.
    H, D = 24, 128
    k, v = _offset_keys(60 + T, T, H, D)
    announce(f"K/V pair at the capacity boundary: {T} tokens, smooth={smooth}, adaptive={adaptive}")
    gpu = nv.KVCache(T, H, D, max_chunks=1, smooth_k=smooth)
    gpu.append(bf16_to_dev(k), bf16_to_dev(v), adaptive46=adaptive)
    ko, vo = gpu.dequant(0, T)
    torch.cuda.synchronize()
    ref = oracle.KVCacheRef(T, H, D, smooth_k=smooth)
    ref.append(k, v, adaptive46=adaptive)
    if smooth:
        _compare(gpu, ref, T)
    else:
        for a, b in ((gpu.k_codes, ref.k_codes), (gpu.v_codes, ref.v_codes), (gpu.k_scales, ref.k_scales),
                     (gpu.v_scales, ref.v_scales)):
            assert np.array_equal(to_np(a)[:T], b[:T])
        assert np.array_equal(to_np(gpu.gscale)[:1], np.array(ref.gscale, dtype=np.float32).reshape(-1, 2))
    rk, rv = ref.dequant(0, T)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)


def test_smoothed_strided_append_and_qkv_append():
    H, D, T = 24, 128, 300
    hd = H * D
    rows = workloads.random_matrix(31, T, 3 * hd, sigma=2.0, outliers=True)
    gpu = nv.KVCache(T, H, D, max_chunks=2, smooth_k=True)
    dev_rows = bf16_to_dev(rows)
    gpu.append(dev_rows[:, hd:2 * hd], dev_rows[:, 2 * hd:])
    ref = oracle.KVCacheRef(T, H, D, smooth_k=True)
    ref.append(np.ascontiguousarray(rows[:, hd:2 * hd]).reshape(T, H, D),
               np.ascontiguousarray(rows[:, 2 * hd:]).reshape(T, H, D))
    torch.cuda.synchronize()
    _compare(gpu, ref, T)
    # the QKV projection with its K and V appended to a smoothed cache
    rng = np.random.default_rng(5)
    w = workloads.to_bf16_bits((rng.standard_normal((3 * hd, 3072)) * 0.02).astype(np.float32))
    b = workloads.to_bf16_bits((rng.standard_normal(3 * hd) + 2).astype(np.float32))   # offsets in K
    x = workloads.to_bf16_bits(rng.standard_normal((200, 3072)).astype(np.float32))
    wq, ws_, wg = nv.quantize(bf16_to_dev(w))
    announce("smoothed qkv_append against linear + smoothed append")
    fused = nv.KVCache(400, H, D, max_chunks=2, smooth_k=True)
    plain = nv.KVCache(400, H, D, max_chunks=2, smooth_k=True)
    for part in (x[:120], x[120:]):
        xd = bf16_to_dev(part)
        q1 = fused.qkv_append(xd, wq, ws_, wg, bias=bf16_to_dev(b), adaptive46=True)
        q2 = nv.linear(xd, wq, ws_, wg, bias=bf16_to_dev(b))
        plain.append(q2[:, hd:2 * hd], q2[:, 2 * hd:], adaptive46=True)
        torch.cuda.synchronize()
        assert torch.equal(q1, q2)
    for name in ("k_codes", "k_scales", "v_codes", "v_scales", "gscale", "chunk_start", "k_center"):
        assert torch.equal(getattr(fused, name), getattr(plain, name)), name


def _smoothed_caches(seed, sizes, H, D=128):
    cap = sum(sizes)
    gpu = nv.KVCache(cap, H, D, max_chunks=len(sizes), smooth_k=True)
    ref = oracle.KVCacheRef(cap, H, D, smooth_k=True)
    for i, T in enumerate(sizes):
        k, v = _offset_keys(seed + i, T, H, D)
        gpu.append(bf16_to_dev(k), bf16_to_dev(v))
        ref.append(k, v)
    return gpu, ref


def _check(o_bits, o64, o_ref_bits, label):
    got = oracle.bf16_bits_to_f32(o_bits).astype(np.float64)
    ref = oracle.bf16_bits_to_f32(o_ref_bits).astype(np.float64)
    for h in range(o64.shape[1]):
        e64 = np.linalg.norm(got[:, h] - o64[:, h]) / np.linalg.norm(o64[:, h])
        eref = np.linalg.norm(got[:, h] - ref[:, h]) / np.linalg.norm(ref[:, h])
        announce(f"  {label} head {h}: {e64:.3e} vs fp64, {eref:.3e} vs bf16 oracle")
        assert e64 <= ATTN_TOL and eref <= ATTN_TOL_BF16, (label, h, e64, eref)


@pytest.mark.parametrize("sizes,Tq,ranges", [
    ([40, 70, 33], 50, [(0, 143)]),                                     # tiles over 2-3 appends
    ([5, 1, 17, 8, 3, 90, 2, 30], 129, [(0, 10), (12, 100), (120, 156)]),   # many short appends, 3 ranges
    ([64, 64], 1, [(5, 6)]),                                            # one query, one key
    ([880, 880, 880, 880, 880, 416], 200, [(0, 880), (2640, 4816)]),    # sink + window, several splits
])
def test_smoothed_attention_against_oracle(sizes, Tq, ranges):
    H = 3
    announce(f"smoothed attention sizes={sizes} Tq={Tq} ranges={ranges}")
    gpu, ref = _smoothed_caches(17, sizes, H)
    rng = np.random.default_rng(18)
    q = workloads.to_bf16_bits((0.3 * rng.standard_normal((Tq, H, 128))).astype(np.float32))
    o = gpu.attention(bf16_to_dev(q), ranges)
    torch.cuda.synchronize()
    o64, oref = oracle.kv_attention_ref(q, ref, ranges)
    _check(to_bits(o), o64, oref, "smoothed")
