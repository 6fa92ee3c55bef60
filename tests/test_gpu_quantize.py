"""GPU parity of nvfp4_quantize: codes, scales and the tensor scale must match
the oracle bit for bit (and the hand-worked golden example)."""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_np

pytestmark = pytest.mark.gpu


def _check(x_bits, label, rows=None, amax=None):
    announce(f"quantize {label} shape={x_bits.shape}")
    codes, scales, g = nv.quantize(bf16_to_dev(x_bits))
    torch.cuda.synchronize()
    c, s, gv = to_np(codes), to_np(scales), to_np(g)[0]
    if rows is None:
        rc, rs, rg = oracle.quantize(x_bits)
        c_cmp, s_cmp = c, s
    else:
        rc, rs, rg = oracle.quantize(x_bits[rows], amax=amax)
        c_cmp, s_cmp = c[rows], s[rows]
    assert np.float32(gv) == rg, (label, gv, rg)
    bad_s = np.argwhere(s_cmp != rs)
    assert bad_s.size == 0, (label, "scales differ at", bad_s[:5])
    bad_c = np.argwhere(c_cmp != rc)
    assert bad_c.size == 0, (label, "codes differ at", bad_c[:5], c_cmp[tuple(bad_c[0])], rc[tuple(bad_c[0])])
    return codes, scales, g


def test_hand_worked_example(golden):
    g = golden("quantize_hand_example.txt")
    rows = [[float(v) for v in g[r]] + [float(v) for v in g[r + "b"]] for r in ("row0", "row1", "row2")]
    x = workloads.to_bf16_bits(np.array(rows, np.float32))
    codes, scales, gs = nv.quantize(bf16_to_dev(x))
    c, s = to_np(codes), to_np(scales)
    assert to_np(gs)[0] == float(g["g"][0])
    for i in range(3):
        assert list(s[i]) == [int(v, 16) for v in g[f"scales{i}"]], i
        assert list(c[i]) == [int(v, 16) for v in g[f"codes{i}"]], i


def test_tiny_config():
    w = workloads.tiny()
    _check(w.x, "tiny X")
    _check(w.w, "tiny W")


@pytest.mark.parametrize("M,K,seed", [(1, 32, 1), (3, 96, 2), (300, 416, 3), (257, 1056, 4),
                                      (5, 4096, 5), (1000, 64, 6), (33, 14336, 7)])
def test_ragged_shapes(M, K, seed):
    _check(workloads.random_matrix(seed, M, K, sigma=2.0, outliers=True), f"random {M}x{K}")


def test_edge_values():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0, :16] = 0.0                                   # all-zero block
    x[1, :16] = -0.0                                  # negative zeros
    x[2, :16] = 1e-40                                 # bf16 subnormals (tiny blocks → S = 0)
    x[2, 16:32] = np.float32(2.0 ** -126) * rng.standard_normal(16).astype(np.float32)
    x[3, :] *= 1e-6                                   # underflowing block scales
    x[4, 0] = 3.0e4                                   # tensor amax (outlier)
    _check(workloads.to_bf16_bits(x), "edge values")


def test_exact_midpoints():
    # A = 168 → g = 2^-4 exactly; the block amax 6·2^-4 gives S = 1.0 and
    # r = 16 exactly, so q lands exactly on every E2M1 midpoint
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 168.0
    mids = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                     -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 5.5], np.float32)
    x[1, :16] = mids / 16
    x[1, 16:] = -mids / 16
    codes, scales, g = _check(workloads.to_bf16_bits(x), "exact midpoints")
    assert to_np(scales)[1, 0] == 0x38 and to_np(g)[0] == 0.0625


def test_all_zero_and_domain_floor():
    z = np.zeros((8, 64), np.uint16)
    z[3, 5] = 0x8000
    _check(z, "all zero")
    x = np.zeros((4, 64), np.float32)
    x[1, 7] = 2.0 ** -100
    x[2, 9] = -(2.0 ** -101)
    _check(workloads.to_bf16_bits(x), "domain floor")


def test_qkv_activation_full():
    w = workloads.qkv()
    _check(w.x, "QKV X [4096,3072] full")


def test_qkv_weight_full():
    w = workloads.qkv()
    _check(w.w, "QKV W [9216,3072] full")


def test_long_context_sampled_rows():
    w = workloads.long_ctx()
    A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()
    rows = np.r_[0:64, 16320:16448, np.random.default_rng(3).integers(0, w.M, 256), w.M - 64:w.M]
    _check(w.x, "long X [32768,3072] sampled rows", rows=np.unique(rows), amax=A)


def test_ffn_hidden_shape_sampled_rows():
    # the down projection's input has shape [8192, 14336]; the quantiser is
    # checked at that full shape on a GELU-like synthetic input
    rng = np.random.default_rng(22)
    h = rng.standard_normal((8192, 14336), dtype=np.float32) * 0.7
    h = np.where(h > 0, h, 0.05 * h).astype(np.float32)
    hb = workloads.to_bf16_bits(h)
    del h
    A = np.abs(oracle.bf16_bits_to_f32(hb)).max()
    rows = np.unique(np.r_[0:32, rng.integers(0, 8192, 200), 8160:8192])
    _check(hb, "H-shaped [8192,14336] sampled rows", rows=rows, amax=A)


@pytest.mark.parametrize("M,K,seed", [(11000, 3072, 51), (81000, 416, 52)])
def test_streamed_beyond_register_capacity(M, K, seed):
    # just past what 256 workgroups x 1024 threads x 8 blocks hold: the first
    # blocks stay in registers, the rest is streamed (read twice); whole-tensor
    # bit-exactness, standard and adaptive, and with the wait forced to expire
    x = workloads.random_matrix(seed, M, K, 1.0, outliers=True)
    _check(x, f"streamed {M}x{K}")
    codes, scales, g = nv.quantize(bf16_to_dev(x), adaptive46=True)
    rc, rs, rg = oracle.quantize(x, adaptive46=True)
    torch.cuda.synchronize()
    assert to_np(g)[0] == rg and np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc)
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    try:
        _check(x, f"streamed {M}x{K}, wait 0")
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)


def test_deterministic():
    w = workloads.qkv()
    x = bf16_to_dev(w.x)
    a = nv.quantize(x)
    b = nv.quantize(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_bounded_wait_fallback_gives_the_same_bytes():
    # force every workgroup of the single-launch quantiser onto the fallback
    # (its own read of the whole tensor) from the host; the bytes must not change
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    try:
        x = workloads.random_matrix(41, 1024, 3072, sigma=1.5, outliers=True)
        _check(x, "random 1024x3072, wait 0")
        codes, scales, g = nv.quantize(bf16_to_dev(x), adaptive46=True)
        rc, rs, rg = oracle.quantize(x, adaptive46=True)
        torch.cuda.synchronize()
        assert to_np(g)[0] == rg and np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc)
        # two tensors in one launch (a KV append)
        rng = np.random.default_rng(42)
        k = workloads.to_bf16_bits(rng.standard_normal((100, 24, 128)).astype(np.float32))
        v = workloads.to_bf16_bits(3 * rng.standard_normal((100, 24, 128)).astype(np.float32))
        kv = nv.KVCache(100, 24, 128, max_chunks=1)
        kv.append(bf16_to_dev(k), bf16_to_dev(v))
        ref = oracle.KVCacheRef(100, 24, 128)
        ref.append(k, v)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(kv.k_codes), ref.k_codes) and np.array_equal(to_np(kv.v_scales), ref.v_scales)
        assert np.array_equal(to_np(kv.gscale)[0], np.array(ref.gscale[0], dtype=np.float32))
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)
    assert L.nvfp4_testing_set_quantize_wait(prev) == prev
