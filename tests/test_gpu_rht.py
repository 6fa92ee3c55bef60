"""GPU parity of nvfp4_quantize_rht (random Hadamard transform of a
weight-gradient operand, then NVFP4 quantisation of its transpose) against the
oracle (oracle/rht.py): codes, scales and the tensor scale bit-exact, at sizes
that span several 256-token × 128-feature tiles with ragged tails, at the FFN
weight-gradient size on sampled feature rows (with the oracle's tensor amax
over the whole transform), and the weight gradient through the W4A4 GEMM
within the GEMM tolerance of the oracle product.
"""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import GEMM_TOL, announce, bf16_to_dev, gemm_errors, to_bits, to_np

pytestmark = pytest.mark.gpu


def _strided(bits, ld):
    """bf16 [T, N] on the device as a view with row stride ld (>= N)."""
    T, N = bits.shape
    full = np.zeros((T, ld), dtype=np.uint16)
    full[:, :N] = bits
    return bf16_to_dev(full)[:, :N]


def _check(x_bits, mask, ld=None):
    T, N = x_bits.shape
    ld = ld or N
    codes, scales, g = nv.quantize_rht(_strided(x_bits, ld), mask)
    torch.cuda.synchronize()
    rc, rs, rg = oracle.quantize_rht(x_bits, mask)
    gc, gs = to_np(codes), to_np(scales)
    bad = np.argwhere((gc != rc).any(axis=1) | (gs != rs).any(axis=1)).ravel()
    assert bad.size == 0, f"{bad.size} feature rows differ, first {bad[:8]}"
    assert to_np(g)[0].view(np.uint32) == np.float32(rg).view(np.uint32)


def _heavy(seed, T, N):
    rng = np.random.default_rng(seed)
    tok = np.exp(rng.standard_normal((T, 1)) * 0.7)
    return workloads.to_bf16_bits((rng.standard_t(4, (T, N)) * tok).astype(np.float32))


@pytest.mark.parametrize("T,N,ld,mask", [
    (512, 300, 304, 0x5DC8),       # 2 x 3 tiles, ragged feature tile (44 of 128, 4 of 8 in a thread)
    (96, 130, 136, 0xFFFF),        # one partial token tile, features 128 + 2
    (32, 1, 8, 0x0001),            # the smallest operand
    (768, 256, 256, 0x0000),       # whole tiles, identity signs
])
def test_quantize_rht_matches_oracle(T, N, ld, mask):
    announce(f"quantize_rht T={T} N={N} ld={ld} mask={mask:#06x}")
    _check(_heavy(T * 7 + N, T, N), mask, ld)


def test_quantize_rht_hand_example(golden):
    g = golden("rht_hand_example.txt")
    T, N = int(g["T"][0]), int(g["N"][0])
    x = np.zeros((T, N), dtype=np.float32)
    for item in g["nonzero_inputs"]:
        t, n, v = item.split(",")
        x[int(t), int(n)] = float(v)
    x[16:32, 1] = float(g["constant_column_1_group_1"][0])
    announce("quantize_rht hand example")
    codes, scales, gs = nv.quantize_rht(_strided(workloads.to_bf16_bits(x), 8), int(g["sign_mask"][0], 16))
    torch.cuda.synchronize()
    assert to_np(gs)[0].view(np.uint32) == int(g["g_bits"][0], 16)
    for n in range(N):
        assert to_np(codes)[n].tolist() == [int(v, 16) for v in g[f"codes_row{n}"]], n
        assert to_np(scales)[n].tolist() == [int(v, 16) for v in g[f"scales_row{n}"]], n


def test_quantize_rht_zeros_and_signed_zeros():
    # an all-zero operand (g = 1, every code +0 under any signs); then zero
    # groups, -0 inputs and exactly cancelling groups next to non-zero data
    announce("quantize_rht zeros")
    codes, scales, g = nv.quantize_rht(bf16_to_dev(np.zeros((64, 24), np.uint16)), 0xFFFF)
    torch.cuda.synchronize()
    assert not to_np(codes).any() and not to_np(scales).any() and to_np(g)[0] == 1.0
    x = np.zeros((64, 24), dtype=np.float32)
    x[:16, :8] = -0.0
    x[16:32, 8:16] = np.r_[1.0, 1.0, np.zeros(14)][:, None]
    x[32:, 16:] = np.random.default_rng(3).standard_normal((32, 8))
    _check(workloads.to_bf16_bits(x), 0xFFFF)


def test_quantize_rht_repeat_and_dense_wide():
    # the same workspace twice (its partials are rewritten before they are
    # read) on a dense operand of 16 x 72 tiles
    x = _heavy(21, 4096, 9216)
    announce("quantize_rht 4096 x 9216, twice with one workspace")
    xd = bf16_to_dev(x)
    ws = torch.empty((nv.quantize_rht_workspace_bytes(4096, 9216),), dtype=torch.uint8, device="cuda")
    first = [to_np(t) for t in nv.quantize_rht(xd, 0x1357, ws=ws)]
    second = [to_np(t) for t in nv.quantize_rht(xd, 0x1357, ws=ws)]
    assert all(np.array_equal(a, b) for a, b in zip(first, second))
    rows = np.unique(np.r_[0:3, np.random.default_rng(1).integers(0, 9216, 24), 9213:9216])
    A = max(float(np.abs(oracle.rht(x[:, c:c + 1024], 0x1357)).max()) for c in range(0, 9216, 1024))
    y = oracle.rht(np.ascontiguousarray(x[:, rows]), 0x1357)
    rc, rs, rg = oracle.quantize_f32(np.ascontiguousarray(y.T), amax=A)
    assert np.array_equal(first[0][rows], rc) and np.array_equal(first[1][rows], rs)
    assert first[2][0] == rg


def test_quantize_rht_full_size_sampled():
    # the FFN up-projection's weight-gradient operands at full size, checked on
    # sampled feature rows against the oracle with its whole-tensor amax
    w = workloads.wgrad()
    for name, x, chunk in (("X", w.x, 512), ("dY", w.dy, 1024)):
        T, N = x.shape
        announce(f"quantize_rht full size {name} [{T}, {N}] mask={w.sign_mask:#06x}")
        codes, scales, g = nv.quantize_rht(bf16_to_dev(x), w.sign_mask)
        torch.cuda.synchronize()
        A = max(float(np.abs(oracle.rht(x[:, c:c + chunk], w.sign_mask)).max()) for c in range(0, N, chunk))
        rows = np.unique(np.r_[0:4, np.random.default_rng(N).integers(0, N, 28), N - 4:N])
        y = oracle.rht(np.ascontiguousarray(x[:, rows]), w.sign_mask)
        rc, rs, rg = oracle.quantize_f32(np.ascontiguousarray(y.T), amax=A)
        assert to_np(g)[0] == rg
        assert np.array_equal(to_np(codes[rows]), rc) and np.array_equal(to_np(scales[rows]), rs)
        del codes, scales


def test_weight_grad_against_oracle():
    # dW = dYᵀ·X through two transformed operands and the W4A4 GEMM
    w = workloads.wgrad(seed=6, T=1024, O=640, I=384)
    announce("weight_grad 640 x 384 over 1024 tokens")
    dW = nv.weight_grad(bf16_to_dev(w.dy), bf16_to_dev(w.x), w.sign_mask)
    torch.cuda.synchronize()
    c64, cref = oracle.gemm_ref(*oracle.quantize_rht(w.dy, w.sign_mask), *oracle.quantize_rht(w.x, w.sign_mask))
    e_ref, e64 = gemm_errors(to_bits(dW), c64, cref)
    assert e_ref <= GEMM_TOL and e64 <= GEMM_TOL, (e_ref, e64)
