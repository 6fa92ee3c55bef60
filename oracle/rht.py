"""Random Hadamard transform before the weight-gradient quantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io reading
notes), 二、方法 / NVFP4 训练的工程细节: gradients use 1-D block scales, and on
the gradient path the operands of the weight-gradient GEMM pass through a
random Hadamard transform before they are quantised, to even out their
distribution.

The weight gradient of a linear layer y = x·Wᵀ over T tokens is
dW[o, i] = Σ_t dy[t, o] · x[t, i], a product whose contraction runs over the
tokens.  The GEMM takes both operands with the contraction axis contiguous, so
each is quantised as its transpose ([features, T], 16-blocks along T).

Readings taken where the pages are silent:
  R29 the transform acts along the contraction (token) axis, on consecutive
      groups of 16 tokens starting at token 0, the size of an NVFP4 block, so
      each block of the quantised transpose is the transform of one group;
  R30 it is R = H₁₆ · diag(s) / 4: H₁₆ the Sylvester Hadamard matrix
      (H[i, k] = (−1)^popcount(i & k)), s a vector of 16 random signs drawn
      by the caller and passed in as a bit mask (bit k set: s_k = −1); the
      same R on every group and on both operands, so that
      Σ_t (R·dy)[t, o] (R·x)[t, i] = Σ_t dy[t, o] x[t, i] (R is orthogonal);
  R31 the transformed values are exact sums of ±bf16 inputs divided by 4,
      rounded once to binary32 (nearest-even), an exactly zero value as +0
      (the sign of an exact zero is an artefact of the summation order and of
      sign flips on zero inputs, so it is fixed); the tensor amax and every
      quantisation decision then follow the binary32 steps of the NVFP4
      quantiser on those values.  (The exact sum of a group is representable
      in binary64 whenever its 16 inputs span less than 2^41 in magnitude,
      which this module assumes and checks.)
  R32 the token count is a multiple of 32 (the GEMM's contraction
      granularity); a caller with another count appends zero tokens, which
      add nothing to the weight gradient.

Parity status: hadamard pinned (scipy.linalg.hadamard, H·Hᵀ = 16·I);
rht pinned (exact rational brute force on small inputs, inverse transform,
invariance of the contraction, a group that is constant along the tokens,
hand-worked signed deltas in tests/golden/rht_hand_example.txt);
quantize_rht pinned (the hand-worked example's codes and scales; quantize_f32
equals the pinned quantize on bf16 values); the evening-out itself pinned (a
spike spreads flat, Student-t tails fall to the kurtosis of a 16-term sum).
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32
from .nvfp4 import BLOCK, quantize_f32

GROUP = 16           # R29: Hadamard size = NVFP4 block size


def hadamard(n: int = GROUP) -> np.ndarray:
    """Sylvester's Hadamard matrix of order n (a power of two), as float64:
    H₁ = [1], H₂ₘ = [[Hₘ, Hₘ], [Hₘ, −Hₘ]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def signs(sign_mask: int) -> np.ndarray:
    """R30: the 16 signs, s_k = −1 where bit k of the mask is set."""
    if not 0 <= int(sign_mask) < (1 << GROUP):
        raise ValueError("sign_mask has 16 bits")
    return np.array([-1.0 if (int(sign_mask) >> k) & 1 else 1.0 for k in range(GROUP)])


def rht_f64(x: np.ndarray, sign_mask: int) -> np.ndarray:
    """R·x on every group of 16 consecutive rows of x [T, N] (any real array),
    in binary64, R = H₁₆·diag(s)/4."""
    x = np.asarray(x, dtype=np.float64)
    T, N = x.shape
    if T % GROUP:
        raise ValueError("T must be a multiple of 16")
    R = hadamard() @ np.diag(signs(sign_mask)) / 4.0
    groups = x.reshape(T // GROUP, GROUP, N)
    return np.einsum("ik,gkn->gin", R, groups).reshape(T, N)


def rht(x_bits: np.ndarray, sign_mask: int) -> np.ndarray:
    """R31: the transform of a bf16 matrix [T, N] (uint16 patterns) along its
    rows, rounded once to binary32.  Returns float32 [T, N]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("x must be 2-D [T, N]")
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    T, N = x.shape
    if T % GROUP:
        raise ValueError("T must be a multiple of 16")
    a = np.abs(x).reshape(T // GROUP, GROUP, N)
    top = a.max(axis=1)
    low = np.where(a > 0, a, np.inf).min(axis=1)
    if np.any((top > 0) & (top >= low * 2.0 ** 41)):
        raise ValueError("a group spans 2^41 or more; its binary64 sum may round (R31)")
    y = rht_f64(x, sign_mask) + 0.0                      # exact in binary64; −0 → +0
    return y.astype(np.float32)                           # one rounding


def quantize_rht(x_bits: np.ndarray, sign_mask: int):
    """The weight-gradient operand: transform x [T, N] along T (R29-R31), then
    NVFP4-quantise its transpose [N, T] with 16-blocks along T.

    Returns ``(codes u8 [N, T/2], scales u8 [N, T/16], g float32)``."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.shape[0] % (2 * BLOCK):
        raise ValueError("T must be a multiple of 32 (R32)")
    y = rht(x_bits, sign_mask)
    return quantize_f32(np.ascontiguousarray(y.T))
