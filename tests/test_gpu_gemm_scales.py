"""GPU parity of the GEMM over the whole E4M3 block-scale range.

The format ("LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 量化格式)
fixes FP8 E4M3 as the block-scale format, so every finite byte 0x00..0x7E is
a valid scale, including the subnormals 0x01..0x07 (m·2^-9).  The kernel
decodes each element to E2M1·S in fp16, which is exact for every code and
every finite scale, and multiplies by selection matrices here so each output
is one such product:

  * exhaustive decode: every one of the 16 codes under every one of the 127
    finite scale bytes, on the activation side and on the weight side, checked
    bit for bit against the oracle;
  * random codes with scale bytes drawn uniformly from 0x00..0x7E, within the
    normwise bound;
  * rows whose blocks all get subnormal scales from the quantiser, next to an
    outlier row, checked row by row (a normwise check over the whole matrix
    would not see them).
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import GEMM_TOL, announce, bf16_to_dev, f32_to_dev, gemm_errors, to_bits, u8_to_dev

pytestmark = pytest.mark.gpu

K_EX = 2048                       # 128 blocks: 127 finite scale bytes + one more


def _pattern(rows, shift):
    """Codes [rows, K_EX/2] and scales [rows, K_EX/16]: in row m, block b has scale byte
    (b + shift·m) mod 127 and its 16 elements carry the codes (c + m) mod 16, so
    every row holds all 16 codes under all 127 finite scale bytes."""
    b = np.arange(K_EX // 16)
    m = np.arange(rows)[:, None]
    scales = ((b[None, :] + shift * m) % 127).astype(np.uint8)
    c = (np.arange(K_EX)[None, :] % 16 + m) % 16
    return oracle.pack_nibbles(c.astype(np.uint8)), scales


def _selection(n):
    """Codes and scales of an [n, K_EX] matrix whose row j is the unit vector e_j
    (E2M1 1.0 = code 0x2 under scale byte 0x38 = 1.0; every other scale 0)."""
    c = np.zeros((n, K_EX), np.uint8)
    c[np.arange(n), np.arange(n)] = 0x2
    s = np.zeros((n, K_EX // 16), np.uint8)
    s[np.arange(n), np.arange(n) // 16] = 0x38
    return oracle.pack_nibbles(c), s


def _values(bits):
    return oracle.bf16_bits_to_f32(bits)        # ±0 compare equal as floats


@pytest.mark.parametrize("ga,gw", [(1.0, 1.0), (3.0, 0.75)])
def test_exhaustive_decode_activation_side(ga, gw):
    # C[m, n] = A[m, n] · fl32(ga·gw): one E2M1·E4M3 product per output, exact in
    # binary32, then one bf16 rounding on both sides
    announce(f"exhaustive E2M1 x E4M3 decode, activation side, g={ga}x{gw}")
    M = 64
    aq, asc = _pattern(M, 3)
    wq, wsc = _selection(K_EX)
    _, cref = oracle.gemm_ref(aq, asc, np.float32(ga), wq, wsc, np.float32(gw))
    out = nv.gemm(u8_to_dev(aq), u8_to_dev(asc), f32_to_dev(ga), u8_to_dev(wq), u8_to_dev(wsc), f32_to_dev(gw))
    torch.cuda.synchronize()
    got = to_bits(out)
    bad = np.argwhere(_values(got) != _values(cref))
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], cref[tuple(bad[0])])
    # the subnormal scale bytes really occur and give nonzero outputs
    sub = (asc[:, :, None].repeat(16, axis=2).reshape(M, K_EX) <= 7) & (asc[:, :, None].repeat(16, axis=2).reshape(M, K_EX) >= 1)
    assert np.count_nonzero(_values(got)[sub]) > 1000


def test_exhaustive_decode_weight_side():
    announce("exhaustive E2M1 x E4M3 decode, weight side")
    N = 96
    wq, wsc = _pattern(N, 5)
    aq, asc = _selection(K_EX)               # A = identity rows: C[m, n] = W[n, m]
    _, cref = oracle.gemm_ref(aq, asc, np.float32(1.0), wq, wsc, np.float32(1.0))
    out = nv.gemm(u8_to_dev(aq), u8_to_dev(asc), f32_to_dev(1.0), u8_to_dev(wq), u8_to_dev(wsc), f32_to_dev(1.0))
    torch.cuda.synchronize()
    got = to_bits(out)
    bad = np.argwhere(_values(got) != _values(cref))
    assert bad.size == 0, (bad[:5], got[tuple(bad[0])], cref[tuple(bad[0])])


@pytest.mark.parametrize("M,N,K,seed", [(300, 260, 512, 1), (513, 777, 1056, 2)])
def test_random_codes_uniform_scale_bytes(M, N, K, seed):
    announce(f"random codes, scale bytes uniform in 0x00..0x7E, {M}x{N}x{K}")
    rng = np.random.default_rng(seed)
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)
    wsc = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    ga, gw = np.float32(0.0123), np.float32(0.00041)
    c64, cref = oracle.gemm_ref(aq, asc, ga, wq, wsc, gw)
    out = nv.gemm(u8_to_dev(aq), u8_to_dev(asc), f32_to_dev(ga), u8_to_dev(wq), u8_to_dev(wsc), f32_to_dev(gw))
    torch.cuda.synchronize()
    e_ref, e_64 = gemm_errors(to_bits(out), c64, cref)
    announce(f"  normwise err vs bf16 oracle {e_ref:.3e}, vs fp64 {e_64:.3e}")
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL


@pytest.mark.parametrize("amax", [2688.0, 1000.0])
def test_subnormal_scale_rows_next_to_an_outlier(amax):
    # One outlier row sets the tensor amax A; the other rows are small enough
    # that every block scale a/(6g) falls in E4M3's subnormal range
    # (a < 2^-6 · 6g).  The GPU quantiser must give the oracle's bytes, and
    # the GEMM's output rows must each be within the bound of the oracle's.
    M, N, K = 200, 320, 1024
    announce(f"subnormal-scale rows next to an outlier row, A={amax}")
    rng = np.random.default_rng(int(amax))
    g = amax / 2688.0
    hi = 0.9 * 2.0 ** -6 * 6 * g
    x = (rng.uniform(0.05, 1.0, (M, K)) * rng.choice([-1, 1], (M, K)) * hi).astype(np.float32)
    x[7] = rng.standard_normal(K).astype(np.float32)
    x[7, 100] = amax
    xb = workloads.to_bf16_bits(x)
    wb = workloads.random_matrix(77, N, K, 0.02)
    qa = oracle.quantize(xb)
    small_rows = np.r_[0:7, 8:M]
    assert qa[1][small_rows].max() <= 7 and np.count_nonzero(qa[1][small_rows]) > 0.9 * qa[1][small_rows].size
    aq, asc, ag = nv.quantize(bf16_to_dev(xb))
    torch.cuda.synchronize()
    assert np.array_equal(aq.cpu().numpy(), qa[0]) and np.array_equal(asc.cpu().numpy(), qa[1])
    assert ag.cpu().numpy()[0] == qa[2]
    qw = oracle.quantize(wb)
    c64, cref = oracle.gemm_ref(*qa, *qw)
    out = nv.gemm(aq, asc, ag, u8_to_dev(qw[0]), u8_to_dev(qw[1]), f32_to_dev(qw[2]))
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f32(to_bits(out)).astype(np.float64)
    for m in range(M):
        den = np.linalg.norm(c64[m])
        assert den > 0, m
        err = np.linalg.norm(got[m] - c64[m]) / den
        assert err <= GEMM_TOL, (m, err)
