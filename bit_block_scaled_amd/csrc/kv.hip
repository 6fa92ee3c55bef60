// NVFP4 KV-cache dequantisation kernel (gfx950).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座: the
// KV cache is stored quantised per chunk and read back through a dequant
// kernel; 二、方法 / NVFP4 量化格式: Dequant = X^FP4 · α^FP8 · α^FP32.
//
// Each thread turns 32 consecutive elements (16 code bytes, 2 scale bytes) of
// one tensor into 64 bytes of bf16:  out = bf16(fl32(fl32(E2M1·S)·g)), where g
// is the tensor scale of the append that wrote the token (binary search over
// the chunk start offsets).  The E2M1·S product is exact in binary32.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kKvThreads = 256;

__device__ __forceinline__ int64_t chunk_of(const int64_t *starts, int64_t n_chunks, int64_t t) {
  int64_t lo = 0, hi = n_chunks - 1;      // invariant: starts[lo] <= t < starts[hi + 1]
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Two bf16 from the 2 codes of byte SEL of `w`: (E2M1 · s) · g, rounded once
// to binary32 and once to bf16.
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
  const int64_t units_per_token = a.elems_per_token / 32;
  const int64_t base_unit = a.t0 * units_per_token;
  const int64_t units = (a.t1 - a.t0) * units_per_token;
  const u32x4 *codes = reinterpret_cast<const u32x4 *>(a.codes[which]) + base_unit;
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.scales[which]) + base_unit;
  u32x4 *out = reinterpret_cast<u32x4 *>(a.out[which]);
  const int64_t stride = (int64_t)gridDim.x * kKvThreads;
  for (int64_t u = (int64_t)blockIdx.x * kKvThreads + threadIdx.x; u < units; u += stride) {
    const int64_t t = a.t0 + u / units_per_token;
    const float g = a.gscale[2 * chunk_of(a.chunk_start, a.n_chunks, t) + which];
    const u32x4 c = codes[u];
    const uint32_t sb = scales[u];
    const float s0 = e4m3_decode(sb & 0xFFu), s1 = e4m3_decode(sb >> 8);
    out[4 * u + 0] = dequant_dword(c.x, s0, g);
    out[4 * u + 1] = dequant_dword(c.y, s0, g);
    out[4 * u + 2] = dequant_dword(c.z, s1, g);
    out[4 * u + 3] = dequant_dword(c.w, s1, g);
  }
}

hipError_t launch_kv_dequant(const KvDequantArgs &a, hipStream_t stream) {
  const int64_t units = (a.t1 - a.t0) * (a.elems_per_token / 32);
  if (units <= 0) return hipSuccess;
  int64_t blocks = (units + kKvThreads - 1) / kKvThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_kv_dequant, dim3((unsigned)blocks, 2), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
