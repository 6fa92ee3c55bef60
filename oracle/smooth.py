"""K-smoothing of an NVFP4 KV-cache chunk: the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io
reading notes), 二、方法 / 推理底座: each KV chunk is quantised again on its
own, with K-smoothing applied to its keys and an adaptive scale choice.  The
pages name K-smoothing without defining it.  The reading taken here is the
usual one for quantised keys: every channel of the chunk's keys has its
centre (its mean over the chunk's tokens) subtracted before quantisation, and
the centre is kept beside the chunk so that the keys can be restored.  The
centre is shared by all tokens of the chunk, so a channel's offset no longer
widens every 16-element block scale of that channel.

Readings (arithmetic fixed so that the centre is exact and independent of the
order in which tokens are summed):
  R33 centre of head h, channel j of a chunk of T tokens:
        z_t = clamp(round_half_even(K[t,h,j] · 2^24), −2^38, 2^38)
        S   = Σ_t z_t                          (an exact integer, |S| < 2^63)
        μ   = bf16_rne( fl64( fl64(S) / T ) · 2^-24 )
      i.e. the mean on a fixed grid of 2^-24 with each key saturated at
      ±16384, rounded once to binary64 per step and then once to bf16;
  R34 smoothed keys K' = bf16_rne(fl32(K − μ)) (one binary32 subtraction,
      then bf16); K' is quantised like any bf16 tensor (its own tensor scale,
      blocks of 16 along head_dim, the adaptive choice when asked for); V is
      not smoothed;
  R35 read-back: K = bf16(fl32(fl32(fl32(E2M1 · S) · g) + μ)) — the dequant
      chain of an unsmoothed cache, then the centre added in binary32;
  R36 attention over a smoothed cache sees each key exactly as
      E2M1 · S · g + μ (binary64), the unsmoothed definition plus the centre.

Parity status: k_center pinned (exact rational brute force on small chunks
with ties, sub-grid values and saturated keys; the hand-worked tie of the
golden example; constant channels give their value and an exactly zero K';
token-permutation invariance; channel shifts move the centre by the shift);
smooth_keys pinned (hand-worked example; K' = K for a zero centre).
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32, bf16_rne_from_f64

GRID_LOG2 = 24                 # fixed-point grid of the centre sum: 2^-24
CLAMP = 1 << 38                # each key counts at most ±2^38 grid steps (±16384)


def k_center(k_bits: np.ndarray) -> np.ndarray:
    """R33: the centre of each channel of a chunk's keys.

    ``k_bits`` [T, H, D] bf16 bit patterns (T >= 1); returns the centres as
    bf16 bit patterns [H, D]."""
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    if k_bits.ndim != 3 or k_bits.shape[0] < 1:
        raise ValueError("keys must be [T >= 1, H, D]")
    T = k_bits.shape[0]
    if T > (1 << 24):
        raise ValueError("a chunk holds at most 2^24 tokens")
    x = bf16_bits_to_f32(k_bits).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("keys must be finite")
    z = np.rint(np.ldexp(x, GRID_LOG2))                      # exact scaling, then ties to even
    z = np.clip(z, -CLAMP, CLAMP).astype(np.int64)           # exact integers
    S = z.sum(axis=0, dtype=np.int64)                        # exact: |S| <= 2^62
    mean = S.astype(np.float64) / np.float64(T)              # fl64(fl64(S) / T)
    return bf16_rne_from_f64(np.ldexp(mean, -GRID_LOG2))


def smooth_keys(k_bits: np.ndarray, mu_bits: np.ndarray) -> np.ndarray:
    """R34: bf16_rne(fl32(K − μ)) for keys [T, H, D] and centres [H, D]."""
    k = bf16_bits_to_f32(np.asarray(k_bits, dtype=np.uint16))
    mu = bf16_bits_to_f32(np.asarray(mu_bits, dtype=np.uint16))
    d = (k - mu[None, :, :]).astype(np.float32)              # one binary32 rounding
    return bf16_rne_from_f64(d.astype(np.float64))           # exact widening, one bf16 rounding
