"""NVFP4 quantise / dequantise, the W4A4 GEMM reference and the NVFP4 KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io
reading notes):
  * 二、方法 / NVFP4 量化格式 — three-level scaling: an FP32 tensor scale that
    normalises the overall range, one FP8 E4M3 scale per 16-element block that
    aligns the local range, and the E2M1 element; dequantisation equation
    Dequant(X) = X^FP4 · α^FP8 · α^FP32.
  * 二、方法 / NVFP4 训练的工程细节 — W4A4 with 1-D block scaling for
    activations; reductions and normalisation stay in higher precision (here:
    FP32 accumulation, FP32 epilogue).
  * 二、方法 / 推理底座 — weights materialised once in 4 bits; the KV cache is
    quantised again per chunk, from 4·T_c·H·d to 9/8·T_c·H·d bytes.

Where the pages leave a step open, the readings taken are:
  R3  tensor scale g = A / (6·448), A = max|x| (the largest block scale lands
      on the top of the E4M3 range);                        [parity unpinned]
  R4  a block's amax maps to the largest E2M1 magnitude 6;
  R5  block scale rounded to nearest-even E4M3, saturating; [parity unpinned]
  R6  elements rounded to nearest-even E2M1, saturating at ±6;
  R7  the element is multiplied by the reciprocal of the dequantisation
      scale, r = 1/(S·g), not divided by it;                [parity unpinned]
  R8  the sign of zero is kept (−0.0 and negatives that round to 0 give 0x8);
  R9  element 2j sits in the low nibble of byte j;          [parity unpinned]
  R10 a block whose scale rounds to 0 encodes all elements as ±0;
  R11 an all-zero tensor gets g = 1;
  R12 inputs are finite and A is 0 or >= 2^-100;
  R15 the KV cache keeps one g per append call per tensor.  [parity unpinned]
  R23 adaptive block scales (二、方法 / 推理底座 and the distillation paragraph of
      二、方法 name an "adaptive scale" search over the amax targets {4, 6}):
      each block is encoded twice, with its amax mapped to 6 (as above) and
      to 4 (divisor fl(4·g) in place of fl(6·g)); the encoding whose block
      squared error is smaller is kept, ties to 6;
  R24 that error is computed in binary32, element by element in index order:
      deq = fl(fl(E2M1·S)·g) with the code's sign, e = fl(x − deq),
      err = fl(err + fl(e·e)) from err = 0.            [parity unpinned]
  R25 two-dimensional weight blocks (二、方法 / NVFP4 训练的工程细节: weights
      scaled in blocks along two dimensions, so W and its transpose share one
      quantisation): a block is 16 consecutive rows (groups from row 0; the
      last group may be shorter) by 16 consecutive elements along K; its
      amax is the largest |x| of the tile, and every row of the tile stores
      the tile's scale byte, so the [M, K/16] scale layout is unchanged.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import (
    E2M1_VALUES,
    bf16_bits_to_f32,
    bf16_rne_from_f64,
    e2m1_rne_sat,
    e4m3_decode,
    e4m3_encode_rne_satfinite,
    pack_nibbles,
    unpack_nibbles,
)
from .smooth import k_center, smooth_keys

BLOCK = 16                      # elements per E4M3 block scale
E2M1_MAX = 6.0                  # largest E2M1 magnitude
E4M3_MAX = 448.0                # largest finite E4M3 value
GLOBAL_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)   # 2688, exact in binary32


def _encode_blocks(blocks, g, target, a_blk=None):
    """Scale bytes and E2M1 magnitude codes of blocks [M, nb, 16] (|x|, binary32)
    with each block's amax mapped to ``target`` (6 or 4): the steps R4-R7, R10.
    ``a_blk`` [M, nb] overrides the per-block amax (two-dimensional blocks)."""
    div = np.float32(np.float32(target) * g)                 # fl(target·g)
    if a_blk is None:
        a_blk = blocks.max(axis=2)                           # exact
    s_raw = (a_blk / div).astype(np.float32)                 # fl(a / (target·g))
    S = e4m3_encode_rne_satfinite(s_raw.astype(np.float64))  # RNE, satfinite
    S_val = e4m3_decode(S).astype(np.float32)                # exact in f32
    d = (S_val * g).astype(np.float32)                       # fl(S·g)
    with np.errstate(divide="ignore"):
        r = np.where(S == 0, np.float32(0.0), (np.float32(1.0) / d)).astype(np.float32)
    q = (blocks * r[:, :, None]).astype(np.float32)          # fl(|x|·r)
    m = e2m1_rne_sat(q.astype(np.float64))
    return S.astype(np.uint8), m.astype(np.uint8)


def block_sq_error(x, S, m, neg, g):
    """R24: per-block squared error of an encoding, in binary32, in index order.

    ``x`` [M, nb, 16] float32 values, ``S`` [M, nb] scale bytes, ``m`` [M, nb, 16]
    magnitude codes, ``neg`` [M, nb, 16] sign flags, ``g`` the tensor scale."""
    S_val = e4m3_decode(S).astype(np.float32)
    mag = E2M1_VALUES[m].astype(np.float32)
    deq = ((mag * S_val[:, :, None]).astype(np.float32) * np.float32(g)).astype(np.float32)
    deq = np.where(neg, -deq, deq).astype(np.float32)
    e = (x - deq).astype(np.float32)
    err = np.zeros(S.shape, dtype=np.float32)
    for i in range(BLOCK):
        err = (err + (e[:, :, i] * e[:, :, i]).astype(np.float32)).astype(np.float32)
    return err


def tile_amax_2d(ax: np.ndarray) -> np.ndarray:
    """R25: for |x| [M, K] (binary32), the amax of each 16x16 tile, repeated on
    every row of the tile: [M, K/16]."""
    M, K = ax.shape
    a1 = ax.reshape(M, K // BLOCK, BLOCK).max(axis=2)        # per row and column block
    groups = (M + BLOCK - 1) // BLOCK
    padded = np.zeros((groups * BLOCK, K // BLOCK), dtype=ax.dtype)
    padded[:M] = a1                                          # |x| >= 0: padding never wins
    a2 = padded.reshape(groups, BLOCK, K // BLOCK).max(axis=1)
    return np.repeat(a2, BLOCK, axis=0)[:M]


def quantize(x_bits: np.ndarray, amax=None, adaptive46=False, blocks2d=False):
    """NVFP4-quantise a bf16 matrix ``x`` [M, K] (given as uint16 bit patterns).

    Returns ``(codes u8 [M, K/2], scales u8 [M, K/16], g float32)``.

    Rows are independent once the tensor amax A is known, so a caller may pass
    a subset of a tensor's rows together with ``amax`` = that tensor's A.
    ``adaptive46`` selects, per block, the better of the amax→6 and amax→4
    encodings (R23, R24); ``blocks2d`` scales 16x16 tiles (R25); the output
    format is unchanged either way (the two options exclude each other).

    The steps, in binary32 (each line one IEEE operation, nearest-even):
      A = max |x|                              (exact)
      g = A / 2688                             (R3)
      per block of 16 along K:  a = max |x|;  S = E4M3(a / (6·g))   (R4, R5)
      d = decode(S) · g;  r = 1/d  (r = 0 when S = 0)                (R7, R10)
      per element: m = E2M1(|x| · r);  code = sign(x)·8 | m          (R6, R8)
      byte j of a row = code[2j] | code[2j+1] << 4                   (R9)
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    return quantize_f32(bf16_bits_to_f32(x_bits), amax, adaptive46, blocks2d)


def quantize_f32(x: np.ndarray, amax=None, adaptive46=False, blocks2d=False):
    """The steps of ``quantize`` on binary32 values ``x`` [M, K] (any binary32,
    not only bf16-representable ones); ``quantize`` is this function applied
    to the bf16 inputs widened exactly to binary32."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    if adaptive46 and blocks2d:
        raise ValueError("adaptive46 and blocks2d exclude each other")
    if blocks2d and amax is not None:
        raise ValueError("blocks2d needs the whole tensor (tiles span rows)")
    M, K = x.shape
    if K % BLOCK or K % 2:
        raise ValueError("K must be a multiple of 16")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite (R12)")
    sign = np.signbit(x).astype(np.uint8) << np.uint8(3)
    ax = np.abs(x)                                           # float32, exact
    A = np.float32(ax.max()) if ax.size else np.float32(0.0)
    if amax is not None:
        if np.float32(amax) < A:
            raise ValueError("amax is smaller than the rows' own maximum")
        A = np.float32(amax)

    if A == 0:                                               # R11
        g = np.float32(1.0)
        scales = np.zeros((M, K // BLOCK), dtype=np.uint8)
        codes = pack_nibbles(sign)
        return codes, scales, g
    if A < np.float32(2.0 ** -100):
        raise ValueError("tensor amax below 2^-100 is outside the domain (R12)")

    g = np.float32(A / GLOBAL_DIVISOR)                       # fl(A / 2688)

    blocks = ax.reshape(M, K // BLOCK, BLOCK)
    S, m = _encode_blocks(blocks, g, E2M1_MAX, tile_amax_2d(ax) if blocks2d else None)
    if adaptive46:
        S4, m4 = _encode_blocks(blocks, g, 4.0)
        xb = x.reshape(M, K // BLOCK, BLOCK)
        neg = (sign.reshape(M, K // BLOCK, BLOCK) != 0)
        e6 = block_sq_error(xb, S, m, neg, g)
        e4 = block_sq_error(xb, S4, m4, neg, g)
        use4 = e4 < e6                                       # ties keep 6
        S = np.where(use4, S4, S).astype(np.uint8)
        m = np.where(use4[:, :, None], m4, m).astype(np.uint8)
    code = (sign | m.reshape(M, K)).astype(np.uint8)
    return pack_nibbles(code), S, g


def dequantize(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """Dequant(X) = X^FP4 · α^FP8 · α^FP32, exactly, in binary64. [M, K]."""
    c = unpack_nibbles(codes)
    M, K = c.shape
    mag = E2M1_VALUES[c & 7]
    val = np.where((c & 8) != 0, -mag, mag)
    s = e4m3_decode(scales).astype(np.float64)
    s = np.repeat(s, BLOCK, axis=1)
    if s.shape != (M, K):
        raise ValueError("scales shape does not match codes")
    return val * s * np.float64(g)


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    """Tanh form of GELU, binary64: 0.5·y·(1 + tanh(√(2/π)·(y + 0.044715·y³)))."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))


def gemm_ref(Aq, As, Ag, Wq, Ws, Wg, bias_bits=None, gelu=False):
    """W4A4 linear layer C = Dequant(A) · Dequant(W)ᵀ (+ bias) (→ GELU).

    A is [M, K] (activations), W is [N, K] (weights, one output row each), both
    NVFP4.  Returns ``(C64 float64 [M, N], C_bf16_bits uint16 [M, N])``: the
    binary64 result and its single nearest-even rounding to bf16.
    """
    a = dequantize(Aq, As, Ag)
    w = dequantize(Wq, Ws, Wg)
    c64 = np.matmul(a, w.T)
    if bias_bits is not None:
        b = bf16_bits_to_f32(bias_bits).astype(np.float64)
        if b.shape != (w.shape[0],):
            raise ValueError("bias must be [N]")
        c64 = c64 + b[None, :]
    if gelu:
        c64 = gelu_tanh(c64)
    return c64, bf16_rne_from_f64(c64)


def gemm_exact_fraction(Aq, As, Ag, Wq, Ws, Wg):
    """Exact rational C = Dequant(A) · Dequant(W)ᵀ with ``fractions.Fraction``.

    Pure-Python loops; for tiny shapes only (used to pin :func:`gemm_ref`).
    """
    ca, cw = unpack_nibbles(Aq), unpack_nibbles(Wq)
    M, K = ca.shape
    N = cw.shape[0]
    e2 = [Fraction(float(v)) for v in E2M1_VALUES]

    def elem(c, s_byte, gv):
        mag = e2[int(c) & 7]
        v = -mag if int(c) & 8 else mag
        return v * Fraction(float(e4m3_decode(s_byte))) * gv

    ga, gw = Fraction(float(Ag)), Fraction(float(Wg))
    A = [[elem(ca[i, k], As[i, k // BLOCK], ga) for k in range(K)] for i in range(M)]
    W = [[elem(cw[j, k], Ws[j, k // BLOCK], gw) for k in range(K)] for j in range(N)]
    return [[sum((A[i][k] * W[j][k] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


# ----------------------------------------------------------------------------
# NVFP4 KV cache
# ----------------------------------------------------------------------------

def kv_bytes(tokens: int, heads: int, head_dim: int, chunks: int = 0) -> int:
    """Bytes held by an NVFP4 K+V cache: codes + block scales (+ 2 f32 per chunk).

    Per tensor, each element costs 1/2 byte of code and 1/16 byte of scale, so
    K and V together cost 2·(9/16)·T·H·d = 9/8·T·H·d bytes (the pages' figure),
    against 2·2·T·H·d = 4·T·H·d for bf16.
    """
    n = tokens * heads * head_dim
    return 2 * (n // 2 + n // BLOCK) + 8 * chunks


class KVCacheRef:
    """Reference NVFP4 KV cache: K and V stored as codes [cap, H, D/2] and
    scales [cap, H, D/16], one (g_K, g_V) pair per append (R15).

    An append of T tokens quantises K and V, each viewed as [T·H, D], with
    :func:`quantize` (blocks of 16 along head_dim) and writes them at the
    current token offset.  With ``smooth_k`` every append first takes the
    centre of each key channel over its tokens and quantises the smoothed
    keys instead (R33, R34, oracle/smooth.py); the centres are kept per
    append in ``k_center`` ([H, D] bf16 bits each) and added back on read.
    """

    def __init__(self, capacity: int, heads: int, head_dim: int, smooth_k: bool = False):
        if head_dim % 32:
            raise ValueError("head_dim must be a multiple of 32")
        self.cap, self.H, self.D = capacity, heads, head_dim
        self.k_codes = np.zeros((capacity, heads, head_dim // 2), np.uint8)
        self.v_codes = np.zeros_like(self.k_codes)
        self.k_scales = np.zeros((capacity, heads, head_dim // BLOCK), np.uint8)
        self.v_scales = np.zeros_like(self.k_scales)
        self.gscale = []          # list of (g_K, g_V) float32
        self.chunk_start = [0]
        self.n_tokens = 0
        self.smooth_k = bool(smooth_k)
        self.k_center = []        # per append: [H, D] bf16 bits (smooth_k only)

    def append(self, k_bits: np.ndarray, v_bits: np.ndarray, adaptive46=False):
        T = k_bits.shape[0]
        if k_bits.shape != (T, self.H, self.D) or v_bits.shape != k_bits.shape:
            raise ValueError("K and V must be [T, H, D]")
        if self.n_tokens + T > self.cap:
            raise ValueError("capacity exceeded")
        n = self.n_tokens
        if self.smooth_k:
            mu = k_center(k_bits)
            self.k_center.append(mu)
            k_bits = smooth_keys(k_bits, mu)
        kc, ks, kg = quantize(k_bits.reshape(T * self.H, self.D), adaptive46=adaptive46)
        vc, vs, vg = quantize(v_bits.reshape(T * self.H, self.D), adaptive46=adaptive46)
        self.k_codes[n:n + T] = kc.reshape(T, self.H, -1)
        self.k_scales[n:n + T] = ks.reshape(T, self.H, -1)
        self.v_codes[n:n + T] = vc.reshape(T, self.H, -1)
        self.v_scales[n:n + T] = vs.reshape(T, self.H, -1)
        self.gscale.append((np.float32(kg), np.float32(vg)))
        self.n_tokens = n + T
        self.chunk_start.append(self.n_tokens)

    def _chunk_of(self, t: np.ndarray) -> np.ndarray:
        return np.searchsorted(np.asarray(self.chunk_start), t, side="right") - 1

    def dequant(self, t0: int, t1: int):
        """bf16 bits of K and V over tokens [t0, t1): [t1-t0, H, D] each.

        Each element is bf16(fl32(fl32(E2M1 · S) · g)): the first product is
        exact in binary32, then one binary32 and one bf16 rounding.  Keys of
        a smoothed cache get their append's centre added in binary32 before
        the bf16 rounding (R35).
        """
        if not (0 <= t0 <= t1 <= self.n_tokens):
            raise ValueError("range outside the filled cache")
        chunk = self._chunk_of(np.arange(t0, t1))
        out = []
        for which, (codes, scales) in enumerate(((self.k_codes, self.k_scales),
                                                 (self.v_codes, self.v_scales))):
            c = unpack_nibbles(codes[t0:t1])                      # [T, H, D]
            mag = E2M1_VALUES[c & 7].astype(np.float32)
            e = np.where((c & 8) != 0, -mag, mag).astype(np.float32)
            s = np.repeat(e4m3_decode(scales[t0:t1]).astype(np.float32), BLOCK, axis=2)
            es = (e * s).astype(np.float32)                       # exact
            g = np.array([self.gscale[ci][which] for ci in chunk], dtype=np.float32)
            v = (es * g[:, None, None]).astype(np.float32)        # fl32(·g)
            if which == 0 and self.smooth_k:
                mu = bf16_bits_to_f32(np.stack([self.k_center[ci] for ci in chunk])
                                      if len(chunk) else np.zeros((0, self.H, self.D), np.uint16))
                v = (v + mu).astype(np.float32)                   # fl32(· + μ)
            out.append(bf16_rne_from_f64(v.astype(np.float64)))
        return out[0], out[1]

    def nbytes(self) -> int:
        return kv_bytes(self.n_tokens, self.H, self.D, len(self.gscale))

    def values(self, tokens) -> tuple:
        """Exact dequantised K and V (binary64) of the given token indices:
        [len(tokens), H, D] each, E2M1 · S · g with the g of each token's
        append (the dequant equation without any rounding), plus the
        append's centre for the keys of a smoothed cache (R36)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        if tokens.size and (tokens.min() < 0 or tokens.max() >= self.n_tokens):
            raise ValueError("token outside the filled cache")
        chunk = self._chunk_of(tokens)
        out = []
        for which, (codes, scales) in enumerate(((self.k_codes, self.k_scales),
                                                 (self.v_codes, self.v_scales))):
            c = unpack_nibbles(codes[tokens])                     # [T, H, D]
            mag = E2M1_VALUES[c & 7]
            e = np.where((c & 8) != 0, -mag, mag)
            s = np.repeat(e4m3_decode(scales[tokens]).astype(np.float64), BLOCK, axis=2)
            g = np.array([self.gscale[ci][which] for ci in chunk], dtype=np.float64)
            val = e * s * g[:, None, None]
            if which == 0 and self.smooth_k and len(chunk):
                val = val + bf16_bits_to_f32(np.stack([self.k_center[ci] for ci in chunk])).astype(np.float64)
            out.append(val)
        return out[0], out[1]
