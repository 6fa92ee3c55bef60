"""CPU oracle for the NVFP4 W4A4 linear layer, the NVFP4 KV cache (with
optional K-smoothing), attention over that cache and the Hadamard-transformed
weight-gradient operands.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP path is checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import it.  The product path (``bit_block_scaled_amd``) never imports, calls or
falls back to anything here, and this package imports nothing from it.

Source of the method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (reading
notes, yingwang.github.io), section 二、方法 / NVFP4 量化格式 — E2M1 elements,
one FP8 E4M3 scale per 16 elements, one FP32 scale per tensor, and the
dequantisation equation Dequant(X) = X^FP4 · α^FP8 · α^FP32; section 二、方法 /
推理底座 — W4A4 inference and the NVFP4 KV cache (4·T_c·H·d → 9/8·T_c·H·d bytes).

Precision: the quantiser runs in IEEE binary32 (the pages fix the tensor scale
as FP32; every code decision is taken in the same precision as the kernel).
Dequantisation and the GEMM run in binary64, where every dequantised value and
product is exact or carries only binary64 rounding.

Parity status per function:
  formats.e2m1_*         pinned (bit-field table, brute-force nearest-even)
  formats.e4m3_*         pinned (exhaustive decode, encode vs torch float8_e4m3fn)
  formats.bf16_*         pinned (torch cast on f32 inputs, hand double-rounding cases)
  nvfp4.quantize         pinned (hand-worked golden block, lossless round trip,
                         amax→±6, sign and power-of-two invariances)
  nvfp4.quantize(adaptive46=True), nvfp4.block_sq_error
                         pinned (hand-worked golden blocks with their errors,
                         lossless on the amax→4 grid, never worse than amax→6
                         in binary64, exact-rational choice, invariances)
  nvfp4.quantize(blocks2d=True), nvfp4.tile_amax_2d
                         pinned (hand-worked tiles, W and its transpose give the
                         transposed dequantised values, a group of equal rows
                         reduces to the 1-D result, tile scale >= row scale)
  nvfp4.dequantize       pinned (dequant equation on round-trip inputs)
  nvfp4.gemm_ref         pinned (Fraction brute force, unit-scale special case,
                         global-scale linearity, block-sum form)
  nvfp4.gelu_tanh        pinned (gelu(0)=0, gelu(y)-gelu(-y)=y, large-|y| limits)
  nvfp4.KVCacheRef       pinned (byte closed form from the pages, append ≡ quantize,
                         hand-worked dequant with a non-power-of-two tensor scale)
  nvfp4.quantize_f32     pinned (equals quantize on bf16-representable values; the
                         binary32 steps of quantize on any binary32 input)
  attention.*            pinned (closed forms, torch's scaled_dot_product_attention
                         in float64, lossless-cache identity; see that module)
  rht.*                  pinned (scipy's Hadamard matrix, exact rational brute force,
                         inverse, contraction invariance, hand-worked example; see
                         that module)
  smooth.*, KVCacheRef(smooth_k=True)
                         pinned (exact rational brute force of the centre, hand-worked
                         tie, constant-channel and shift closed forms, permutation
                         invariance, lossless round trip; see that module)
  The choices of global-scale formula, scale rounding mode, reciprocal-multiply
  order, nibble order, per-append KV scale and the binary32 error order of the
  adaptive selection are fixed by definition only
  ("parity unpinned" for those choices; see the readings in the design notes).
"""

from .formats import (
    E2M1_VALUES,
    e2m1_value_of_bits,
    e2m1_rne_sat,
    e4m3_decode,
    e4m3_encode_rne_satfinite,
    bf16_bits_to_f32,
    bf16_rne_from_f64,
    pack_nibbles,
    unpack_nibbles,
)
from .nvfp4 import (
    GLOBAL_DIVISOR,
    quantize,
    quantize_f32,
    block_sq_error,
    tile_amax_2d,
    dequantize,
    gemm_ref,
    gelu_tanh,
    kv_bytes,
    KVCacheRef,
)
from .attention import attention_ref, kv_attention_ref, range_tokens
from .rht import hadamard, rht, rht_f64, quantize_rht
from .smooth import k_center, smooth_keys

__all__ = [
    "E2M1_VALUES",
    "e2m1_value_of_bits",
    "e2m1_rne_sat",
    "e4m3_decode",
    "e4m3_encode_rne_satfinite",
    "bf16_bits_to_f32",
    "bf16_rne_from_f64",
    "pack_nibbles",
    "unpack_nibbles",
    "GLOBAL_DIVISOR",
    "quantize",
    "quantize_f32",
    "block_sq_error",
    "tile_amax_2d",
    "dequantize",
    "gemm_ref",
    "gelu_tanh",
    "kv_bytes",
    "KVCacheRef",
    "attention_ref",
    "kv_attention_ref",
    "range_tokens",
    "hadamard",
    "rht",
    "rht_f64",
    "quantize_rht",
    "k_center",
    "smooth_keys",
]
