"""Attention over an NVFP4 KV cache: the plain definition, in binary64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io reading
notes):
  * 二、方法 / 推理底座 — the KV cache is stored in NVFP4 per chunk and read
    back through a dequantisation kernel inside inference; its overhead is
    stated to stay within 2 %.
  * 二、方法 / 多镜头注意力锚点 — the KV set a chunk attends to is
    A_g ∪ A_s ∪ KV[t − W, t): the global-sink frames, the shot-sink frames and
    a window of recent frames, with duplicates removed.
  * The notes assume the reader knows Transformer attention; the operator is
    the textbook one, softmax(Q·Kᵀ·scale)·V per head.

Readings taken where the pages are silent:
  R26 the keys and values of a query chunk are the cache tokens of a list of
      disjoint token ranges (the sink and window sets as ranges of the cache;
      the caller removes duplicates by passing disjoint ranges); no mask inside
      that set;
  R27 scale = 1/sqrt(head_dim) unless given;
  R28 K and V enter the attention exactly dequantised, E2M1 · S · g per
      element (the dequant equation with no rounding), and the queries are the
      bf16 inputs; the result is rounded once to bf16.

Parity status: attention_ref pinned (uniform scores give the mean of V; one
key gives V; key-permutation invariance; V scaled by 2 gives O scaled by 2;
agreement within 1e-12 with torch's scaled_dot_product_attention in float64
on random inputs, a library routine);
kv_attention_ref pinned (equals attention_ref on the bf16 K/V when the cache
holds them losslessly, including across appends with different tensor scales;
a list of ranges equals the concatenated keys).
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32, bf16_rne_from_f64


def attention_ref(q, k, v, scale=None):
    """softmax(q·kᵀ·scale)·v per head, binary64.

    q [Tq, H, D], k and v [Tk, H, D] (any real arrays; computed in binary64).
    Returns O [Tq, H, D] float64.  Each softmax row subtracts its maximum
    before the exponential (the same value, without overflow)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, H, D = q.shape
    if k.shape[1:] != (H, D) or v.shape != k.shape or k.shape[0] < 1:
        raise ValueError("k and v must be [Tk >= 1, H, D] like q")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((Tq, H, D), dtype=np.float64)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale                     # [Tq, Tk]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def range_tokens(ranges) -> np.ndarray:
    """Token indices of a list of [start, end) ranges, in order (R26)."""
    parts = [np.arange(int(a), int(b), dtype=np.int64) for a, b in ranges]
    t = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    if len(np.unique(t)) != len(t):
        raise ValueError("ranges must be disjoint")
    return t


def kv_attention_ref(q_bits, cache, ranges, scale=None):
    """Attention of bf16 queries [Tq, H, D] (bit patterns) over the tokens of
    `ranges` in an oracle NVFP4 cache (KVCacheRef), keys and values exactly
    dequantised (R26-R28).  Returns (O64 [Tq, H, D] float64, O bf16 bits)."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    k, v = cache.values(range_tokens(ranges))
    o = attention_ref(q, k, v, scale)
    return o, bf16_rne_from_f64(o)
