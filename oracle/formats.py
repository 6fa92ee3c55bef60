"""Element formats of NVFP4, written out from their bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", section 二、方法 /
NVFP4 量化格式 and the 缩写表 entry for NVFP4: the element is E2M1 (1 sign,
2 exponent, 1 mantissa bit); the block scale is FP8 E4M3; the tensor scale is
FP32.  The pages give only the bit split; the exponent biases used here are the
standard ones for these formats (E2M1 bias 1 with a subnormal at exponent 0;
E4M3 in its "FN" form: bias 7, no infinities, NaN only at S.1111.111, largest
finite 448).

Every conversion here is a nearest-value search over the format's value set,
ties to the even encoding — the definition of round-to-nearest-even — rather
than bit arithmetic, so that it shares no technique with the GPU kernels.
"""

from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# E2M1 (FP4) element
# ----------------------------------------------------------------------------

def e2m1_value_of_bits(m3: int) -> float:
    """Magnitude of the 3 non-sign bits ``e1 e0 m`` of an E2M1 code.

    Exponent bias 1: exponent field 0 is subnormal, value = m/2; otherwise
    value = 2^(e-1) · (1 + m/2).
    """
    e = (m3 >> 1) & 3
    m = m3 & 1
    if e == 0:
        return 0.5 * m
    return float(2.0 ** (e - 1) * (1.0 + 0.5 * m))


#: The 8 magnitudes, indexed by the 3 magnitude bits (derived, not typed in).
E2M1_VALUES = np.array([e2m1_value_of_bits(i) for i in range(8)], dtype=np.float64)


def e2m1_rne_sat(q: np.ndarray) -> np.ndarray:
    """Magnitude bits (0..7) of the E2M1 value nearest to ``q`` (q >= 0).

    Ties go to the code whose mantissa bit is 0 (even).  Values above the
    largest magnitude 6 saturate to 6 (code 7).
    """
    q = np.asarray(q, dtype=np.float64)
    if np.any(q < 0) or np.any(~np.isfinite(q)):
        raise ValueError("e2m1_rne_sat expects finite non-negative magnitudes")
    vals = E2M1_VALUES
    lo = np.searchsorted(vals, q, side="right") - 1          # largest value <= q
    lo = np.clip(lo, 0, 7)
    hi = np.clip(lo + 1, 0, 7)
    d_lo = q - vals[lo]
    d_hi = vals[hi] - q
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    out = np.where(pick_hi, hi, lo)
    out = np.where(q >= vals[7], 7, out)                       # saturate
    return out.astype(np.uint8)


# ----------------------------------------------------------------------------
# E4M3 (FP8, "FN" variant) block scale
# ----------------------------------------------------------------------------

def _e4m3_decode_scalar(b: int) -> float:
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        v = m * 2.0 ** -9
    else:
        v = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -v if s else v


_E4M3_TABLE = np.array([_e4m3_decode_scalar(b) for b in range(256)], dtype=np.float64)
# Non-negative finite values in byte order 0x00..0x7E; strictly increasing.
_E4M3_POS = _E4M3_TABLE[:0x7F]


def e4m3_decode(b) -> np.ndarray:
    """Value of E4M3 byte(s) as float64 (exact)."""
    return _E4M3_TABLE[np.asarray(b, dtype=np.uint8)]


def e4m3_encode_rne_satfinite(v) -> np.ndarray:
    """E4M3 byte nearest to ``v`` (v >= 0), ties to even, saturating at 448.

    Consecutive bytes 0x00..0x7E are consecutive representable values, so the
    byte with an even mantissa LSB is simply the even byte.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(~np.isfinite(v)):
        raise ValueError("e4m3 encode expects finite non-negative values")
    vals = _E4M3_POS
    lo = np.clip(np.searchsorted(vals, v, side="right") - 1, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    d_lo = v - vals[lo]
    d_hi = vals[hi] - v
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    out = np.where(pick_hi, hi, lo)
    out = np.where(v >= vals[0x7E], 0x7E, out)                 # satfinite
    return out.astype(np.uint8)


# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) → float32, exact (bf16 is the top half of f32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_rne_from_f64(x) -> np.ndarray:
    """bf16 bit patterns of the bf16 value nearest to each finite ``x``.

    One rounding, from the exact binary64 value: 8 significant bits for
    normals (|x| >= 2^-126), a fixed quantum 2^-133 below that; ties to even.
    Overflow beyond the largest finite bf16 raises (never reached here).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)):
        raise ValueError("bf16_rne_from_f64 expects finite values")
    ax = np.abs(x)
    _, ex = np.frexp(ax)                   # ax = f · 2^ex, f in [0.5, 1)
    lead = ex - 1                          # exponent of the leading bit
    quantum_exp = np.where(lead >= -126, lead - 7, -133)
    n = np.ldexp(ax, -quantum_exp)         # exact power-of-two scaling
    r = np.rint(n)                         # round half to even
    val = np.ldexp(r, quantum_exp)
    max_bf16 = float.fromhex("0x1.fep127")
    if np.any(val > max_bf16):
        raise OverflowError("value beyond the bf16 range")
    val = np.where(np.signbit(x), -val, val)
    f32 = val.astype(np.float32)           # exact: val has <= 8 significant bits
    if not np.array_equal(f32.astype(np.float64), val):
        raise AssertionError("internal: rounded value not representable")
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Nibble packing (reading: element 2j sits in the low nibble of byte j)
# ----------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes → [..., n] bytes, element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("need an even number of codes")
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
