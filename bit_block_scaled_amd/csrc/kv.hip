// NVFP4 KV-cache dequantisation kernel (gfx950).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座: the
// KV cache is stored quantised per chunk and read back through a dequant
// kernel; 二、方法 / NVFP4 量化格式: Dequant = X^FP4 · α^FP8 · α^FP32.
//
// Layout of the work: every lane turns one 8-element group (4 code bytes, one
// scale byte shared with its neighbour lane) into 16 bytes of bf16, so each
// load and store instruction of a wave covers consecutive memory; a thread
// handles kKvU groups, kKvThreads apart.  out = bf16(fl32(fl32(E2M1·S)·g)),
// where g is the tensor scale of the append that wrote the token (the E2M1·S
// product is exact in binary32); keys of a K-smoothed cache get their
// append's channel centre added in binary32 before the bf16 rounding.
//
// Finding each token's append: a wave covers few tokens (under 3 for 24
// heads of 128), so it first brackets its token range: the appends holding
// its first and its last token, each found by a 64-wide search (every lane
// compares one chunk start, a ballot counts the starts at or below the token;
// one round per 64 appends).  Then each lane searches only inside that
// bracket, which is usually a single append.  The starts are read from global
// memory (they stay in the caches); no LDS, no barrier.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kKvThreads = 256;
constexpr int kKvU = 4;                    // 8-element groups per thread

// Index of the append holding token t (starts[c] <= t < starts[c + 1]),
// computed by the whole wave for a wave-uniform t: the number of starts
// starts[1..n_chunks-1] that are <= t.
__device__ __forceinline__ int64_t chunk_of_uniform(const int64_t *starts, int64_t n_chunks, int64_t t) {
  const int lane = threadIdx.x & 63;
  int64_t c = 0;
  for (int64_t base = 1; base < n_chunks; base += 64) {
    const int64_t j = base + lane;
    const bool le = j < n_chunks && starts[j] <= t;
    const int n = __builtin_popcountll(__ballot(le));
    c += n;
    if (n < 64) break;                       // starts are increasing: no later one is <= t
  }
  return c;
}

// Index of the append holding token t, knowing it lies in [lo, hi].
__device__ __forceinline__ int64_t chunk_in(const int64_t *starts, int64_t lo, int64_t hi, int64_t t) {
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Eight bf16 from the 8 codes of `w`: (E2M1 · s) · g, rounded once to
// binary32 and once to bf16.
template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t w, float s, float g) {
  const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return pack_bf16x2((e.x * s) * g, (e.y * s) * g);
}

__device__ __forceinline__ u32x4 dequant_dword(uint32_t w, float s, float g) {
  u32x4 o;
  o.x = dequant_pair<0>(w, s, g);
  o.y = dequant_pair<1>(w, s, g);
  o.z = dequant_pair<2>(w, s, g);
  o.w = dequant_pair<3>(w, s, g);
  return o;
}

// Keys of a K-smoothed cache: the same chain, then the append's channel
// centre added in binary32 (a separate rounding, never fused with the
// product) before the bf16 rounding.
template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair_centred(uint32_t w, float s, float g, uint32_t mu2) {
#pragma clang fp contract(off)
  const f32x2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const float a = (e.x * s) * g, b = (e.y * s) * g;
  return pack_bf16x2(a + bf16_bits_to_f32(mu2 & 0xFFFFu), b + bf16_bits_to_f32(mu2 >> 16));
}

__device__ __forceinline__ u32x4 dequant_dword_centred(uint32_t w, float s, float g, const u32x4 &mu) {
  u32x4 o;
  o.x = dequant_pair_centred<0>(w, s, g, mu.x);
  o.y = dequant_pair_centred<1>(w, s, g, mu.y);
  o.z = dequant_pair_centred<2>(w, s, g, mu.z);
  o.w = dequant_pair_centred<3>(w, s, g, mu.w);
  return o;
}

__global__ void __launch_bounds__(kKvThreads) k_kv_dequant(KvDequantArgs a) {
  const int which = blockIdx.y;
  const int64_t e = a.elems_per_token;
  const int64_t base = a.t0 * e / 8;                 // first group of the range
  const int64_t groups = (a.t1 - a.t0) * e / 8;
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(a.codes[which]) + base;
  const uint8_t *scales = a.scales[which] + base / 2;
  u32x4 *out = reinterpret_cast<u32x4 *>(a.out[which]);
  const bool narrow = 8 * (groups + kKvThreads * kKvU) < (int64_t(1) << 32);   // 32-bit token division

  // loads first, so the append search below overlaps them
  uint32_t c[kKvU], sb[kKvU];
  int64_t q[kKvU];
#pragma unroll
  for (int i = 0; i < kKvU; ++i) {
    q[i] = ((int64_t)blockIdx.x * kKvU + i) * kKvThreads + threadIdx.x;
    c[i] = q[i] < groups ? codes[q[i]] : 0u;
    sb[i] = q[i] < groups ? scales[q[i] >> 1] : 0u;
  }
  auto token = [&](int64_t g) {
    return a.t0 + (narrow ? (int64_t)((uint32_t)(8 * g) / (uint32_t)e) : (8 * g) / e);
  };
  // the wave's groups: q[0] of its lane 0 to q[kKvU-1] of its lane 63
  const int64_t w0 = q[0] - (threadIdx.x & 63);
  int64_t w1 = w0 + (int64_t)(kKvU - 1) * kKvThreads + 63;
  if (w1 >= groups) w1 = groups - 1;
  if (w0 >= groups) return;                           // the whole wave is past the range
  const int64_t c_lo = chunk_of_uniform(a.chunk_start, a.n_chunks, token(w0));
  const int64_t c_hi = chunk_of_uniform(a.chunk_start, a.n_chunks, token(w1));
#pragma unroll
  for (int i = 0; i < kKvU; ++i) {
    if (q[i] >= groups) continue;
    const int64_t ci = c_lo == c_hi ? c_lo : chunk_in(a.chunk_start, c_lo, c_hi, token(q[i]));
    const float g = a.gscale[2 * ci + which];
    u32x4 o;
    if (which == 0 && a.kcenter != nullptr) {
      const int64_t ch = 8 * q[i] - (token(q[i]) - a.t0) * e;        // channel of the group
      const u32x4 mu = *reinterpret_cast<const u32x4 *>(a.kcenter + ci * e + ch);
      o = dequant_dword_centred(c[i], e4m3_decode(sb[i]), g, mu);
    } else {
      o = dequant_dword(c[i], e4m3_decode(sb[i]), g);
    }
    // non-temporal: the output streams past L2 and the MALL
    __builtin_nontemporal_store(o, &out[q[i]]);
  }
}

hipError_t launch_kv_dequant(const KvDequantArgs &a, hipStream_t stream) {
  const int64_t groups = (a.t1 - a.t0) * (a.elems_per_token / 8);
  if (groups <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)kKvThreads * kKvU;
  const int64_t blocks = (groups + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kv_dequant, dim3((unsigned)blocks, 2), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
