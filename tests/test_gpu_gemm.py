"""GPU parity of nvfp4_gemm / nvfp4_linear against the oracle's FP64 GEMM.

Operands are quantised by the oracle on the CPU (from seeded bf16 inputs) and
uploaded, so the GEMM is checked on exactly the oracle's codes.  The output must
be within 2e-3 normwise of both the bf16-rounded oracle result and the
unrounded FP64 result.  The full-size linear layer (GPU quantiser + GEMM, the
product path) is checked on sampled rows and columns.
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import (GEMM_TOL, announce, bf16_to_dev, f32_to_dev, gemm_errors, to_bits,
                         u8_to_dev)

pytestmark = pytest.mark.gpu


def _upload_q(q):
    c, s, g = q
    return u8_to_dev(c), u8_to_dev(s), f32_to_dev(g)


def _run(M, N, K, seed, bias=False, gelu=False, tile=None, sigma_x=1.0):
    announce(f"gemm M={M} N={N} K={K} seed={seed} bias={bias} gelu={gelu} tile={tile}")
    x = workloads.random_matrix(seed, M, K, sigma_x, outliers=True)
    w = workloads.random_matrix(seed + 1000, N, K, 0.02)
    b = workloads.random_matrix(seed + 2000, 1, N, 0.01)[0] if bias else None
    qa, qw = oracle.quantize(x), oracle.quantize(w)
    c64, cref = oracle.gemm_ref(*qa, *qw, bias_bits=b, gelu=gelu)
    out = nv.gemm(*_upload_q(qa), *_upload_q(qw), bias=None if b is None else bf16_to_dev(b),
                  gelu=gelu, tile=tile)
    torch.cuda.synchronize()
    e_ref, e_64 = gemm_errors(to_bits(out), c64, cref)
    announce(f"  normwise err vs bf16 oracle {e_ref:.3e}, vs fp64 {e_64:.3e}")
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL, (e_ref, e_64)
    return e_ref, e_64


def test_tiny_config():
    w = workloads.tiny()
    qa, qw = oracle.quantize(w.x), oracle.quantize(w.w)
    c64, cref = oracle.gemm_ref(*qa, *qw)
    out = nv.gemm(*_upload_q(qa), *_upload_q(qw))
    torch.cuda.synchronize()
    e_ref, e_64 = gemm_errors(to_bits(out), c64, cref)
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL
    # FP32 accumulation of exact products: beyond bf16 rounding, only a few
    # results may sit one bf16 step away from the oracle's rounding
    diff = np.abs(to_bits(out).astype(np.int32) - cref.astype(np.int32))
    assert diff.max() <= 1 and (diff > 0).mean() < 0.01


@pytest.mark.parametrize("M,N,K,seed", [(300, 200, 416, 1), (1, 1, 32, 2), (1, 8, 64, 3),
                                        (77, 333, 160, 4), (513, 257, 1024, 5), (64, 64, 14336, 6)])
def test_ragged(M, N, K, seed):
    _run(M, N, K, seed, bias=True)


@pytest.mark.parametrize("tile", [(256, 256), (256, 192), (192, 256), (256, 128), (128, 256), (128, 128)])
def test_every_tile(tile):
    _run(600, 520, 384, 11, bias=True, tile=tile)


TILES = [(256, 256), (256, 192), (192, 256), (256, 128), (128, 256), (128, 128)]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("K", [384, 416])
@pytest.mark.parametrize("gelu,bias", [(False, False), (False, True), (True, False), (True, True)])
def test_every_kernel_variant(tile, K, gelu, bias):
    """Every compiled kernel: each tile shape, with and without a K tail (K % 128 = 32), GELU and
    bias, on a ragged 300x290 output whose first 3 rows of X are zero (without GELU their outputs
    are the bias alone, or +0.0, bit for bit)."""
    M, N, seed = 300, 290, 21 + K + 2 * gelu + bias
    announce(f"gemm variant tile={tile} K={K} gelu={gelu} bias={bias}")
    x = workloads.random_matrix(seed, M, K, 3.0 if gelu else 1.0, outliers=True)
    x[:3] = 0
    w = workloads.random_matrix(seed + 1000, N, K, 0.02)
    b = workloads.random_matrix(seed + 2000, 1, N, 0.01)[0] if bias else None
    qa, qw = oracle.quantize(x), oracle.quantize(w)
    c64, cref = oracle.gemm_ref(*qa, *qw, bias_bits=b, gelu=gelu)
    out = nv.gemm(*_upload_q(qa), *_upload_q(qw), bias=None if b is None else bf16_to_dev(b),
                  gelu=gelu, tile=tile)
    torch.cuda.synchronize()
    got = to_bits(out)
    e_ref, e_64 = gemm_errors(got, c64, cref)
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL, (e_ref, e_64)
    if not gelu:
        # the zero rows are exactly the oracle's (bias, or +0.0 bit for bit)
        assert np.array_equal(got[:3], cref[:3])
        # away from cancellation (outputs above 1 % of the RMS, where the FP32 accumulation
        # error stays far below a bf16 step) the result is the oracle's bf16 or a neighbour
        vals = oracle.bf16_bits_to_f32(cref).astype(np.float64)
        big = np.abs(vals) >= 1e-2 * np.sqrt(np.mean(vals * vals))
        diff = np.abs(got.astype(np.int32) - cref.astype(np.int32))[big]
        assert diff.max() <= 1 and (diff > 0).mean() < 0.01


def test_gelu_epilogue():
    _run(256, 384, 512, 12, gelu=True, sigma_x=3.0)


def test_bias_and_gelu():
    _run(130, 96, 256, 13, bias=True, gelu=True)


def _sampled_linear(w, rows, cols, gelu=False):
    """GPU linear on the full workload; oracle on sampled rows x columns."""
    x = bf16_to_dev(w.x)
    qw = oracle.quantize(w.w)
    bias = None if w.bias is None else bf16_to_dev(w.bias)
    out = nv.linear(x, *_upload_q(qw), bias=bias, gelu=gelu)
    torch.cuda.synchronize()
    A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()
    qa = oracle.quantize(w.x[rows], amax=A)
    wc = (qw[0][cols], qw[1][cols], qw[2])
    b = None if w.bias is None else w.bias[cols]
    c64, cref = oracle.gemm_ref(*qa, *wc, bias_bits=b, gelu=gelu)
    got = to_bits(out)[np.ix_(rows, cols)]
    return gemm_errors(got, c64, cref)


def test_qkv_linear_full_size_sampled():
    w = workloads.qkv()
    announce("linear QKV 4096x9216x3072 (sampled check)")
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[0:32, rng.integers(0, w.M, 96), w.M - 32:w.M])
    cols = np.unique(np.r_[0:64, rng.integers(0, w.N, 192), w.N - 64:w.N])
    e_ref, e_64 = _sampled_linear(w, rows, cols)
    announce(f"  normwise err vs bf16 oracle {e_ref:.3e}, vs fp64 {e_64:.3e}")
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL


def test_long_linear_full_size_sampled():
    w = workloads.long_ctx()
    announce("linear long 32768x3072x3072 (sampled check)")
    rng = np.random.default_rng(1)
    rows = np.unique(np.r_[0:32, 16368:16400, rng.integers(0, w.M, 64), w.M - 32:w.M])
    cols = np.unique(np.r_[0:32, rng.integers(0, w.N, 96), w.N - 32:w.N])
    e_ref, e_64 = _sampled_linear(w, rows, cols)
    announce(f"  normwise err vs bf16 oracle {e_ref:.3e}, vs fp64 {e_64:.3e}")
    assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL


def test_gemm_deterministic():
    x = workloads.random_matrix(5, 512, 1024)
    w = workloads.random_matrix(6, 768, 1024, 0.02)
    a = _upload_q(oracle.quantize(x))
    b = _upload_q(oracle.quantize(w))
    o1 = nv.gemm(*a, *b)
    o2 = nv.gemm(*a, *b)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
