// NVFP4 KV-cache dequantisation kernel (gfx950).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座: the
// KV cache is stored quantised per chunk and read back through a dequant
// kernel; 二、方法 / NVFP4 量化格式: Dequant = X^FP4 · α^FP8 · α^FP32.
//
// Layout of the work: every lane turns one 8-element chunk (4 code bytes, one
// scale byte shared with its neighbour lane) into 16 bytes of bf16, so each
// load and store instruction of a wave covers consecutive memory; a workgroup
// handles kKvU chunks per lane.  out = bf16(fl32(fl32(E2M1·S)·g)), where g is
// the tensor scale of the append that wrote the token, found by binary search
// over the chunk start offsets (copied to LDS when they fit).  The E2M1·S
// product is exact in binary32.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kKvThreads = 256;
constexpr int kKvU = 4;                    // chunks per lane
constexpr int kKvLdsStarts = 2048;         // chunk starts held in LDS

// Index of the chunk holding token t: starts[lo] <= t < starts[lo + 1].
template <typename P>
__device__ __forceinline__ int64_t chunk_of(P starts, int64_t n_chunks, int64_t t) {
  int64_t lo = 0, hi = n_chunks - 1;
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

__global__ void __launch_bounds__(kKvThreads) k_kv_dequant(KvDequantArgs a) {
  const int which = blockIdx.y;
  const int64_t e = a.elems_per_token;
  const int64_t base = a.t0 * e / 8;                 // first chunk of the range
  const int64_t chunks = (a.t1 - a.t0) * e / 8;
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(a.codes[which]) + base;
  const uint8_t *scales = a.scales[which] + base / 2;
  u32x4 *out = reinterpret_cast<u32x4 *>(a.out[which]);
  const bool narrow = 8 * (chunks + kKvThreads * kKvU) < (int64_t(1) << 32);   // 32-bit token division

  // loads first, so the chunk search below overlaps them
  uint32_t c[kKvU], sb[kKvU];
#pragma unroll
  for (int i = 0; i < kKvU; ++i) {
    const int64_t q = ((int64_t)blockIdx.x * kKvU + i) * kKvThreads + threadIdx.x;
    c[i] = q < chunks ? codes[q] : 0u;
    sb[i] = q < chunks ? scales[q >> 1] : 0u;
  }
  __shared__ int64_t st[kKvLdsStarts];
  const bool in_lds = a.n_chunks < kKvLdsStarts;
  if (in_lds) {
    for (int64_t j = threadIdx.x; j <= a.n_chunks; j += kKvThreads) st[j] = a.chunk_start[j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kKvU; ++i) {
    const int64_t q = ((int64_t)blockIdx.x * kKvU + i) * kKvThreads + threadIdx.x;
    const int64_t t = a.t0 + (narrow ? (int64_t)((uint32_t)(8 * q) / (uint32_t)e) : (8 * q) / e);
    const int64_t ci = in_lds ? chunk_of(st, a.n_chunks, t) : chunk_of(a.chunk_start, a.n_chunks, t);
    const float g = a.gscale[2 * ci + which];
    const u32x4 o = dequant_dword(c[i], e4m3_decode(sb[i]), g);
    // non-temporal: the output streams past L2 and the MALL (measured 5.9 →
    // 7.2 TB/s on a 65536-token read-back)
    if (q < chunks) __builtin_nontemporal_store(o, &out[q]);
  }
}

hipError_t launch_kv_dequant(const KvDequantArgs &a, hipStream_t stream) {
  const int64_t chunks = (a.t1 - a.t0) * (a.elems_per_token / 8);
  if (chunks <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)kKvThreads * kKvU;
  const int64_t blocks = (chunks + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kv_dequant, dim3((unsigned)blocks, 2), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
