"""Seeded synthetic inputs for the NVFP4 linear layer and KV cache.

Shared by the tests, the benchmark and the oracle checks.  This module holds no
quantisation, dequantisation or GEMM arithmetic: it only draws random numbers
and rounds them to bf16 (via torch's float32→bfloat16 cast) so both sides see
identical bit patterns.

Workload shapes follow the DiT linear layers of the video model the source pages
describe ("LongLive-2.0" reading notes, 二、方法 / 推理底座: W4A4 inference of
the DiT, NVFP4 KV cache; the 5B DiT has 24 heads of 128 = 3072 channels):

  tiny   X [128, 256] ~ N(0,1);  W [256, 256] ~ N(0, 0.02);  seed 0
  qkv    X [4096, 3072] ~ N(0,1) with 0.1 % of entries ×50;  W [9216, 3072]
         (Q, K, V stacked) ~ N(0, 0.02);  bias [9216] ~ N(0, 0.01);  seed 1
  ffn    X [8192, 3072] ~ N(0,1) with 0.1 % ×50;  W_up [14336, 3072],
         W_down [3072, 14336] ~ N(0, 0.02);  seed 2
  long   X [32768, 3072]: first 16384 rows (clean history) ~ N(0,1), last
         16384 rows (noisy target) ~ N(0, 1.5);  W [3072, 3072] ~ N(0, 0.02); seed 3
  kv     K, V [65536, 24, 128] ~ N(0,1) × a per-head factor U(0.5, 4)
         (24 draws for K, then 24 for V, constant over tokens), appended in
         74 chunks of 880 tokens and one of 416;  seed 4
  wgrad  weight gradient of the FFN up-projection over T = 8192 tokens:
         dY [T, 14336] ~ N(0, 10^-3) × a per-token factor exp(N(0, 0.5²)),
         X [T, 3072] ~ N(0,1) with 0.1 % ×50; then the 16 random signs of the
         Hadamard transform as a 16-bit mask;  seed 5

σ in N(0, σ) is the standard deviation.  Draw order inside a workload: X, then
W (then W_down), then bias, then outlier positions.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

HEADS = 24
HEAD_DIM = 128
KV_TOKENS = 65536
KV_CHUNK = 880


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array → bf16 bit patterns (uint16), nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _normal(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def _outliers(rng, x: np.ndarray, frac=0.001, factor=50.0):
    n = int(round(frac * x.size))
    pos = rng.choice(x.size, size=n, replace=False)
    flat = x.reshape(-1)
    flat[pos] *= np.float32(factor)
    return x


@dataclass
class LinearWorkload:
    name: str
    seed: int
    x: np.ndarray                 # bf16 bits [M, K]
    w: np.ndarray                 # bf16 bits [N, K]
    bias: np.ndarray | None       # bf16 bits [N] or None
    w2: np.ndarray | None = None  # second weight (FFN down) [K, N]
    gelu: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.w.shape[0]


def tiny(seed: int = 0) -> LinearWorkload:
    rng = np.random.default_rng(seed)
    x = _normal(rng, (128, 256))
    w = _normal(rng, (256, 256), 0.02)
    return LinearWorkload("tiny 128x256x256", seed, to_bf16_bits(x), to_bf16_bits(w), None)


def qkv(seed: int = 1, M: int = 4096) -> LinearWorkload:
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, 3072))
    w = _normal(rng, (3 * 3072, 3072), 0.02)
    b = _normal(rng, (3 * 3072,), 0.01)
    x = _outliers(rng, x)
    return LinearWorkload(f"DiT QKV projection {M}x9216x3072 + bias", seed,
                          to_bf16_bits(x), to_bf16_bits(w), to_bf16_bits(b))


def ffn(seed: int = 2, M: int = 8192) -> LinearWorkload:
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, 3072))
    w_up = _normal(rng, (14336, 3072), 0.02)
    w_down = _normal(rng, (3072, 14336), 0.02)
    x = _outliers(rng, x)
    return LinearWorkload(f"DiT FFN up {M}x14336x3072 (+GELU) then down {M}x3072x14336", seed,
                          to_bf16_bits(x), to_bf16_bits(w_up), None,
                          w2=to_bf16_bits(w_down), gelu=True)


def long_ctx(seed: int = 3, M: int = 32768) -> LinearWorkload:
    rng = np.random.default_rng(seed)
    half = M // 2
    hist = _normal(rng, (half, 3072), 1.0)
    targ = _normal(rng, (M - half, 3072), 1.5)
    x = np.concatenate([hist, targ], axis=0)
    w = _normal(rng, (3072, 3072), 0.02)
    return LinearWorkload(f"long-context out-proj {M}x3072x3072", seed,
                          to_bf16_bits(x), to_bf16_bits(w), None)


def kv_chunk_sizes(tokens: int = KV_TOKENS, chunk: int = KV_CHUNK):
    sizes = [chunk] * (tokens // chunk)
    if tokens % chunk:
        sizes.append(tokens % chunk)
    return sizes


def kv(seed: int = 4, tokens: int = KV_TOKENS, heads: int = HEADS, head_dim: int = HEAD_DIM):
    """K and V as bf16 bits [tokens, heads, head_dim] plus the append sizes."""
    rng = np.random.default_rng(seed)
    fk = rng.uniform(0.5, 4.0, size=heads).astype(np.float32)
    fv = rng.uniform(0.5, 4.0, size=heads).astype(np.float32)
    k = _normal(rng, (tokens, heads, head_dim)) * fk[None, :, None]
    v = _normal(rng, (tokens, heads, head_dim)) * fv[None, :, None]
    return to_bf16_bits(k), to_bf16_bits(v), kv_chunk_sizes(tokens)


@dataclass
class WgradWorkload:
    name: str
    seed: int
    dy: np.ndarray                # bf16 bits [T, O]
    x: np.ndarray                 # bf16 bits [T, I]
    sign_mask: int


def wgrad(seed: int = 5, T: int = 8192, O: int = 14336, I: int = 3072) -> WgradWorkload:
    rng = np.random.default_rng(seed)
    tok = np.exp(rng.standard_normal((T, 1)) * 0.5).astype(np.float32)
    dy = _normal(rng, (T, O), 1e-3) * tok
    x = _outliers(rng, _normal(rng, (T, I)))
    mask = int(rng.integers(0, 1 << 16))
    return WgradWorkload(f"FFN up weight gradient dW [{O}, {I}] = dYᵀ·X over {T} tokens", seed,
                         to_bf16_bits(dy), to_bf16_bits(x), mask)


def random_matrix(seed: int, M: int, K: int, sigma: float = 1.0, outliers: bool = False):
    """A generic seeded bf16 matrix for ragged-shape tests."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (M, K), sigma)
    if outliers and x.size >= 1000:
        x = _outliers(rng, x)
    return to_bf16_bits(x)


BY_NAME = {"tiny": tiny, "qkv": qkv, "ffn": ffn, "long": long_ctx}
