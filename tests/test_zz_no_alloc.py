"""nvfp4_linear_noalloc (the linear layer with the library's built-in device
workspace) against nvfp4_linear with a caller workspace: identical bytes on
two calls in a row, the second with a smaller input, through the C ABI."""

import ctypes as C

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import GEMM_TOL, announce, bf16_to_dev, gemm_errors, to_bits

pytestmark = pytest.mark.gpu


def _call_noalloc(x, wq, ws, wg, bias, out, flags=0):
    M, K = x.shape
    N = wq.shape[0]
    p = lambda t: None if t is None else C.c_void_p(t.data_ptr())
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return nv.lib().nvfp4_linear_noalloc(p(x), p(wq), p(ws), p(wg), p(bias), p(out), M, N, K, flags, st)


def test_noalloc_matches_linear_two_calls_second_smaller():
    cases = [(4096, 3072, 9216, True, 0), (300, 1024, 520, False, nv.NVFP4_EPI_GELU_TANH)]
    for i, (M, K, N, with_bias, flags) in enumerate(cases):
        announce(f"linear_noalloc call {i}: {M}x{N}x{K} bias={with_bias} flags={flags}")
        xb = workloads.random_matrix(200 + i, M, K, 1.0 + i, outliers=True)
        x = bf16_to_dev(xb)
        wq, ws, wg = nv.quantize(bf16_to_dev(workloads.random_matrix(300 + i, N, K, 0.02)))
        bias = bf16_to_dev(workloads.random_matrix(400 + i, 1, N, 0.01)[0]) if with_bias else None
        got = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        assert _call_noalloc(x, wq, ws, wg, bias, got, flags) == 0, nv.lib().nvfp4_last_error()
        want = nv.linear(x, wq, ws, wg, bias=bias, gelu=bool(flags & nv.NVFP4_EPI_GELU_TANH))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), i
        # and within the GEMM bound of the oracle on sampled rows
        rows = np.unique(np.r_[0:8, np.random.default_rng(i).integers(0, M, 24), M - 8:M])
        A = np.abs(oracle.bf16_bits_to_f32(xb)).max()
        qa = oracle.quantize(xb[rows], amax=A)
        qw = (wq.cpu().numpy(), ws.cpu().numpy(), wg.cpu().numpy()[0])
        b = None if bias is None else to_bits(bias)
        c64, cref = oracle.gemm_ref(*qa, *qw, bias_bits=b, gelu=bool(flags))
        e_ref, e_64 = gemm_errors(to_bits(got)[rows], c64, cref)
        assert e_ref <= GEMM_TOL and e_64 <= GEMM_TOL, (i, e_ref, e_64)


def test_noalloc_rejects_beyond_the_limit():
    # the limit is checked on the host before anything is enqueued (the CPU
    # suite checks the same rejection with addresses that are never used);
    # the buffers here have the claimed sizes all the same
    x = torch.empty((nv.NVFP4_NOALLOC_MAX_ELEMENTS // 1024 + 1, 1024), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((32, 512), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((32, 64), dtype=torch.uint8, device="cuda")
    wg = torch.ones((1,), dtype=torch.float32, device="cuda")
    out = torch.empty((x.shape[0], 32), dtype=torch.bfloat16, device="cuda")
    s = _call_noalloc(x, wq, ws, wg, None, out)
    assert s == 1 and b"NVFP4_NOALLOC_MAX_ELEMENTS" in nv.lib().nvfp4_last_error()
