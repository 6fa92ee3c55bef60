// Device helpers shared by the NVFP4 kernels (gfx950 only).
//
// Format facts used here ("LongLive-2.0：用 NVFP4 并行底座做长视频生成",
// 二、方法 / NVFP4 量化格式): elements are E2M1, block scales FP8 E4M3 (one per
// 16 elements), the tensor scale FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr float kGlobalDivisor = 2688.0f;   // 6 (largest E2M1) · 448 (largest E4M3)
constexpr float kE2M1Max = 6.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Nearest-even E4M3 ("FN": bias 7, max 448) encoding of a finite s >= 0, with
// saturation to 448.  Normal range: round the binary32 bit pattern to 3
// mantissa bits (the carry runs into the exponent); below 2^-6 the grid is the
// fixed quantum 2^-9, so the byte is the nearest-even integer of s·2^9.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float s) {
  if (s >= 448.0f) return 0x7Eu;
  if (s < 0.015625f) {                       // 2^-6
    float t = s * 512.0f;                    // exact
    return (uint32_t)__builtin_rintf(t);     // 0..8, 8 = 2^-6 = byte 0x08
  }
  uint32_t u = __float_as_uint(s);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // RNE to 3 mantissa bits
  uint32_t b = r - (120u << 3);              // rebias exponent 127 → 7
  return b > 0x7Eu ? 0x7Eu : b;
}

// E4M3 byte → float (exact), OCP decoding of the hardware converter.
__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// bf16 pair from two floats, nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Largest bf16 magnitude (as its 15-bit pattern) in a dword pair-wise.
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t acc, uint32_t v) {
  typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// Raw buffer descriptor (stride 0, `bytes` addressable bytes from `base`;
// loads past the end return 0).  Every field is made wave-uniform so the
// descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  i32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  d.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(v >> 32) & 0xFFFFu));
  d.z = __builtin_amdgcn_readfirstlane((int)bytes);
  d.w = 0x00020000;                        // descriptor word 3 for the gfx9 family
  __amdgpu_buffer_rsrc_t r;
  __builtin_memcpy(&r, &d, sizeof(r));
  return r;
}

// Per-tensor constants of the block-scale arithmetic.  Both divisions of a
// block are done with FMA refinements that return the correctly rounded
// binary32 result:
//   s_raw = fl(a / 6g): a and 6g are first scaled by the same power of two
//     (exact) so 6g lies in [1, 2); then q0 = a·y with y = fl(1/6g), the
//     residual a − q0·6g (exact by FMA) and q0 + residual·y rounded once give
//     the correctly rounded quotient (Markstein's theorem: y is the correctly
//     rounded reciprocal and q0 lies within one ulp of the quotient; for bf16
//     block maxima an exhaustive CPU check finds no E4M3 byte that differs);
//   r = fl(1/d): one Newton step y0 + y0·(1 − d·y0) from the hardware
//     reciprocal (within 1 ulp) rounds correctly for every binary32
//     significand (checked exhaustively on the CPU).
// The block amax maps to `target` (6, or 4 for the second candidate of the
// adaptive selection), i.e. the divisor is fl(target·g).
struct BlockScaler {
  float g, sc, bs, y;
  __device__ __forceinline__ BlockScaler(float g_, float target) : g(g_) {
    const float div = target * g;                                 // fl(target·g)
    sc = __uint_as_float((254u - ((__float_as_uint(div) >> 23) & 0xFFu)) << 23);   // 2^-e(div)
    bs = div * sc;
    y = 1.0f / bs;
  }
  // E4M3 scale byte of a block whose largest magnitude is a (binary32, >= 0).
  __device__ __forceinline__ uint32_t scale_byte_of(float a) const {
    const float as = a * sc;
    const float q0 = as * y;
    const float res = __builtin_fmaf(-q0, bs, as);
    return e4m3_encode_rne_sat(__builtin_fmaf(res, y, q0));       // fl(a / div) → E4M3
  }
  // The same for a largest magnitude given as its bf16 pattern bm.
  __device__ __forceinline__ uint32_t scale_byte(uint32_t bm) const {
    return scale_byte_of(bf16_bits_to_f32(bm));
  }
  // fl(1 / fl(S·g)), 0 for S == 0.
  __device__ __forceinline__ float recip(uint32_t S) const {
    const float d = e4m3_decode(S) * g;                           // fl(S·g)
    const float y0 = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, y0, 1.0f);
    const float r = __builtin_fmaf(e, y0, y0);
    return S == 0 ? 0.0f : r;
  }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace nvfp4
