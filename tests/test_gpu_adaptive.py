"""GPU parity of the adaptive {4, 6} block-scale mode (nvfp4_quantize_ex and
nvfp4_kv_append_ex with NVFP4_Q_ADAPTIVE_4_6): codes, scales and tensor
scales bit-exact against the oracle and the hand-worked golden tensor, in the
resident (single-launch) and the two-pass quantiser alike."""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_bits, to_np

pytestmark = pytest.mark.gpu


def _check(x_bits, label, rows=None, amax=None):
    announce(f"adaptive quantize {label} shape={x_bits.shape}")
    codes, scales, g = nv.quantize(bf16_to_dev(x_bits), adaptive46=True)
    torch.cuda.synchronize()
    c, s, gv = to_np(codes), to_np(scales), to_np(g)[0]
    if rows is None:
        rc, rs, rg = oracle.quantize(x_bits, adaptive46=True)
    else:
        rc, rs, rg = oracle.quantize(x_bits[rows], amax=amax, adaptive46=True)
        c, s = c[rows], s[rows]
    assert np.float32(gv) == rg, (label, gv, rg)
    bad = np.argwhere(s != rs)
    assert bad.size == 0, (label, "scales differ at", bad[:5])
    bad = np.argwhere(c != rc)
    assert bad.size == 0, (label, "codes differ at", bad[:5])
    return s


def test_hand_worked_example(golden):
    g = golden("quantize_adaptive_hand_example.txt")
    row = [float(v) for k in ("x0", "x1", "x2", "x3") for v in g[k]]
    x = workloads.to_bf16_bits(np.array([row], np.float32))
    for adaptive, sk, ck in ((False, "scales_std", "codes_std"), (True, "scales_ad", "codes_ad")):
        codes, scales, gs = nv.quantize(bf16_to_dev(x), adaptive46=adaptive)
        assert to_np(gs)[0] == float(g["g"][0])
        assert list(to_np(scales)[0]) == [int(v, 16) for v in g[sk]], sk
        assert list(to_np(codes)[0]) == [int(v, 16) for v in g[ck]], ck


@pytest.mark.parametrize("M,K,seed", [(1, 32, 1), (3, 96, 2), (300, 416, 3), (257, 1056, 4),
                                      (1000, 64, 6), (33, 14336, 7)])
def test_ragged_shapes(M, K, seed):
    s = _check(workloads.random_matrix(seed, M, K, sigma=2.0, outliers=True), f"random {M}x{K}")
    assert M * K < 2048 or (s != oracle.quantize(workloads.random_matrix(seed, M, K, sigma=2.0,
                                                                        outliers=True))[1]).any()


def test_four_grid_blocks():
    # blocks on the amax→4 grid: the adaptive encoding is lossless
    rng = np.random.default_rng(5)
    M, K = 64, 256
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4])
    c = rng.choice(grid, size=(M, K // 16, 16)) * rng.choice([-1, 1], size=(M, K // 16, 16))
    c[:, :, 5] = 4.0
    s = oracle.e4m3_decode(rng.integers(8, 0x7F, size=(M, K // 16)))
    x = (c * s[:, :, None] * 2.0 ** -3).reshape(M, K)
    x[0, :16] = 0.0
    x[0, 0] = 2688.0 * 2.0 ** -3
    xb = workloads.to_bf16_bits(x.astype(np.float32))
    _check(xb, "amax→4 grid")
    codes, scales, g = nv.quantize(bf16_to_dev(xb), adaptive46=True)
    assert np.array_equal(oracle.dequantize(to_np(codes), to_np(scales), to_np(g)[0]), x)


def test_qkv_activation_full():
    _check(workloads.qkv().x, "QKV X [4096,3072] full")


def test_qkv_weight_sampled_rows():
    w = workloads.qkv()
    A = np.abs(oracle.bf16_bits_to_f32(w.w)).max()
    rows = np.unique(np.r_[0:64, np.random.default_rng(9).integers(0, w.N, 512), w.N - 64:w.N])
    _check(w.w, "QKV W [9216,3072] sampled rows", rows=rows, amax=A)


def test_long_context_two_pass_sampled_rows():
    # larger than the resident capacity: the two-pass kernels
    w = workloads.long_ctx()
    A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()
    rows = np.unique(np.r_[0:64, np.random.default_rng(4).integers(0, w.M, 256), w.M - 64:w.M])
    _check(w.x, "long X [32768,3072] sampled rows", rows=rows, amax=A)


def _small_kv(seed, T, H, D):
    rng = np.random.default_rng(seed)
    f = rng.uniform(0.5, 4.0, size=H).astype(np.float32)
    k = rng.standard_normal((T, H, D)).astype(np.float32) * f[None, :, None]
    v = rng.standard_normal((T, H, D)).astype(np.float32) * f[::-1][None, :, None] * 3
    return workloads.to_bf16_bits(k), workloads.to_bf16_bits(v)


def test_kv_appends_mixed_modes_and_dequant():
    H, D = 24, 128
    sizes = [(7, True), (33, False), (1, True), (120, True)]
    cap = sum(t for t, _ in sizes)
    gpu = nv.KVCache(cap, H, D, max_chunks=len(sizes))
    ref = oracle.KVCacheRef(cap, H, D)
    for i, (T, ad) in enumerate(sizes):
        announce(f"kv append T={T} adaptive={ad}")
        k, v = _small_kv(40 + i, T, H, D)
        gpu.append(bf16_to_dev(k), bf16_to_dev(v), adaptive46=ad)
        ref.append(k, v, adaptive46=ad)
    torch.cuda.synchronize()
    n = ref.n_tokens
    for a, b, name in ((gpu.k_codes, ref.k_codes, "k_codes"), (gpu.v_codes, ref.v_codes, "v_codes"),
                       (gpu.k_scales, ref.k_scales, "k_scales"), (gpu.v_scales, ref.v_scales, "v_scales")):
        bad = np.argwhere(to_np(a)[:n] != b[:n])
        assert bad.size == 0, (name, bad[:5])
    assert np.array_equal(to_np(gpu.gscale), np.array(ref.gscale, dtype=np.float32).reshape(-1, 2))
    ko, vo = gpu.dequant(0, n)
    rk, rv = ref.dequant(0, n)
    assert np.array_equal(to_bits(ko), rk) and np.array_equal(to_bits(vo), rv)


def test_kv_full_chunk_adaptive():
    # one 880-token append of the KV workload's geometry, adaptive
    K, V, sizes = workloads.kv()
    T = sizes[0]
    announce(f"kv adaptive append of {T} tokens")
    gpu = nv.KVCache(T, workloads.HEADS, workloads.HEAD_DIM, max_chunks=1)
    gpu.append(bf16_to_dev(K[:T]), bf16_to_dev(V[:T]), adaptive46=True)
    ref = oracle.KVCacheRef(T, workloads.HEADS, workloads.HEAD_DIM)
    ref.append(K[:T], V[:T], adaptive46=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(gpu.k_codes), ref.k_codes)
    assert np.array_equal(to_np(gpu.v_codes), ref.v_codes)
    assert np.array_equal(to_np(gpu.k_scales), ref.k_scales)
    assert np.array_equal(to_np(gpu.v_scales), ref.v_scales)
