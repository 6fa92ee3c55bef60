// NVFP4 quantiser kernels (gfx950).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 量化格式
// (E2M1 elements, one E4M3 scale per 16 elements, one FP32 tensor scale) and
// NVFP4 训练的工程细节 (1-D block scaling of activations).  The same kernels
// quantise the KV cache in place (二、方法 / 推理底座).
//
// Two passes over the input:
//   k_amax    grid-stride max of |x| (on the 15-bit magnitude pattern, which
//             orders like the value for finite bf16); one partial per block.
//   k_encode  every block first folds the partials into A and derives
//             g = A/2688; then each thread encodes 32 consecutive elements
//             (two 16-blocks): block amax → E4M3 scale → reciprocal → E2M1
//             codes, written as one 16-byte store plus one 2-byte scale store.
// With K % 32 == 0 a 32-element unit never crosses a row, and the outputs are
// dense in unit order; the input may be row-strided (a KV append can read the
// K and V column slices of a fused QKV output in place).
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kThreads = 256;

// One tensor per blockIdx.y (the KV append quantises K and V in one launch).
struct QuantTensor {
  const uint16_t *x;     // bf16 input
  uint8_t *codes;        // 16 bytes per 32-element unit
  uint16_t *scales;      // 2 scale bytes per unit
  float *gscale;         // where g is written
  uint32_t *partials;    // kAmaxBlocks partial maxima
  int64_t units;         // elements / 32
  uint32_t units_per_row;
  int64_t ld;            // input elements between row starts
};

// First 16-byte chunk of unit u in the (possibly row-strided) input.
__device__ __forceinline__ const u32x4 *unit_src(const QuantTensor &T, int64_t u) {
  const uint32_t row = (uint32_t)u / T.units_per_row;
  const uint32_t col = (uint32_t)u - row * T.units_per_row;
  return reinterpret_cast<const u32x4 *>(T.x + (int64_t)row * T.ld + 32 * (int64_t)col);
}
struct QuantArgs {
  QuantTensor t[2];
  ChunkMark mark;        // chunk_start == nullptr: nothing to record
};

__global__ void __launch_bounds__(kThreads) k_amax(QuantArgs args) {
  const QuantTensor &T = args.t[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m = 0;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + stride < T.units; u += 2 * stride) {
    const u32x4 *p0 = unit_src(T, u), *p1 = unit_src(T, u + stride);
    const u32x4 a0 = p0[0], a1 = p0[1], a2 = p0[2], a3 = p0[3];
    const u32x4 b0 = p1[0], b1 = p1[1], b2 = p1[2], b3 = p1[3];
    m = absmax_bf16x2(m, a0.x); m = absmax_bf16x2(m, a0.y); m = absmax_bf16x2(m, a0.z); m = absmax_bf16x2(m, a0.w);
    m = absmax_bf16x2(m, a1.x); m = absmax_bf16x2(m, a1.y); m = absmax_bf16x2(m, a1.z); m = absmax_bf16x2(m, a1.w);
    m = absmax_bf16x2(m, a2.x); m = absmax_bf16x2(m, a2.y); m = absmax_bf16x2(m, a2.z); m = absmax_bf16x2(m, a2.w);
    m = absmax_bf16x2(m, a3.x); m = absmax_bf16x2(m, a3.y); m = absmax_bf16x2(m, a3.z); m = absmax_bf16x2(m, a3.w);
    m = absmax_bf16x2(m, b0.x); m = absmax_bf16x2(m, b0.y); m = absmax_bf16x2(m, b0.z); m = absmax_bf16x2(m, b0.w);
    m = absmax_bf16x2(m, b1.x); m = absmax_bf16x2(m, b1.y); m = absmax_bf16x2(m, b1.z); m = absmax_bf16x2(m, b1.w);
    m = absmax_bf16x2(m, b2.x); m = absmax_bf16x2(m, b2.y); m = absmax_bf16x2(m, b2.z); m = absmax_bf16x2(m, b2.w);
    m = absmax_bf16x2(m, b3.x); m = absmax_bf16x2(m, b3.y); m = absmax_bf16x2(m, b3.z); m = absmax_bf16x2(m, b3.w);
  }
  for (; u < T.units; u += stride) {
    const u32x4 *p0 = unit_src(T, u);
    const u32x4 a0 = p0[0], a1 = p0[1], a2 = p0[2], a3 = p0[3];
    m = absmax_bf16x2(m, a0.x); m = absmax_bf16x2(m, a0.y); m = absmax_bf16x2(m, a0.z); m = absmax_bf16x2(m, a0.w);
    m = absmax_bf16x2(m, a1.x); m = absmax_bf16x2(m, a1.y); m = absmax_bf16x2(m, a1.z); m = absmax_bf16x2(m, a1.w);
    m = absmax_bf16x2(m, a2.x); m = absmax_bf16x2(m, a2.y); m = absmax_bf16x2(m, a2.z); m = absmax_bf16x2(m, a2.w);
    m = absmax_bf16x2(m, a3.x); m = absmax_bf16x2(m, a3.y); m = absmax_bf16x2(m, a3.z); m = absmax_bf16x2(m, a3.w);
  }
  uint32_t mm = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
  mm = wave_max_u32(mm);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mm;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
    T.partials[blockIdx.x] = r;
  }
}

// Folds the amax partials of one tensor into (g, 6g).  Every block does this.
__device__ __forceinline__ void block_global_scale(const QuantTensor &T, int nparts,
                                                   float &g, float &six_g) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0;
  for (int p = threadIdx.x; p < nparts; p += kThreads) {
    uint32_t v = T.partials[p];
    m = m > v ? m : v;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
  const float A = bf16_bits_to_f32(r);
  g = (r == 0) ? 1.0f : A / kGlobalDivisor;                // fl(A / 2688)
  six_g = kE2M1Max * g;                                      // fl(6·g)
}

// E2M1 codes of the bf16 pair w scaled by r, written into byte SEL of old
// (first element in the low nibble).  The converter rounds to nearest even,
// saturates at ±6 and keeps the sign of zero; its scale operand is 1.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t old, uint32_t w, float r) {
  const float x0 = bf16_bits_to_f32(w & 0xFFFFu), x1 = bf16_bits_to_f32(w >> 16);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0 * r, x1 * r, 1.0f, SEL);
}

// Encodes one 16-element block held as 8 bf16 pairs; returns the scale byte
// and writes the 8 code bytes to lo/hi (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t encode_block16(const uint32_t (&w)[8], float g, float six_g,
                                                   uint32_t &lo, uint32_t &hi) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = absmax_bf16x2(m, w[j]);
  uint32_t mm = (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
  const float a = bf16_bits_to_f32(mm);
  const float s_raw = a / six_g;                             // fl(a / 6g)
  const uint32_t S = e4m3_encode_rne_sat(s_raw);
  const float d = e4m3_decode(S) * g;                        // fl(S·g)
  const float r = (S == 0) ? 0.0f : 1.0f / d;                // fl(1/d)
  uint32_t c0 = 0, c1 = 0;
  c0 = cvt_pair<0>(c0, w[0], r);
  c0 = cvt_pair<1>(c0, w[1], r);
  c0 = cvt_pair<2>(c0, w[2], r);
  c0 = cvt_pair<3>(c0, w[3], r);
  c1 = cvt_pair<0>(c1, w[4], r);
  c1 = cvt_pair<1>(c1, w[5], r);
  c1 = cvt_pair<2>(c1, w[6], r);
  c1 = cvt_pair<3>(c1, w[7], r);
  lo = c0;
  hi = c1;
  return S;
}

__global__ void __launch_bounds__(kThreads) k_encode(QuantArgs args, int nparts) {
  const QuantTensor &T = args.t[blockIdx.y];
  float g, six_g;
  block_global_scale(T, nparts, g, six_g);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *T.gscale = g;
    if (blockIdx.y == 0 && args.mark.chunk_start != nullptr) {
      args.mark.chunk_start[args.mark.index] = args.mark.value;
      if (args.mark.index == 1) args.mark.chunk_start[0] = 0;
    }
  }
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < T.units; u += stride) {
    const u32x4 *src = unit_src(T, u);
    const u32x4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
    uint32_t b0[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t b1[8] = {v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
    uint32_t c0, c1, c2, c3;
    const uint32_t s0 = encode_block16(b0, g, six_g, c0, c1);
    const uint32_t s1 = encode_block16(b1, g, six_g, c2, c3);
    reinterpret_cast<u32x4 *>(T.codes)[u] = u32x4{c0, c1, c2, c3};
    T.scales[u] = (uint16_t)(s0 | (s1 << 8));
  }
}

static int amax_blocks(int64_t units) {
  int64_t b = (units + kThreads * 2 - 1) / (kThreads * 2);        // >= 2 units per thread
  if (b < 1) b = 1;
  if (b > kAmaxBlocks) b = kAmaxBlocks;
  return (int)b;
}

static int encode_blocks(int64_t units) {
  int64_t b = (units + kThreads - 1) / kThreads;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  return (int)b;
}

hipError_t launch_quantize(const QuantJob *jobs, int njobs, hipStream_t stream,
                           const ChunkMark *mark) {
  QuantArgs a{};
  if (mark) a.mark = *mark;
  int64_t max_units = 0;
  for (int i = 0; i < njobs; ++i) {
    a.t[i].x = jobs[i].x;
    a.t[i].codes = jobs[i].codes;
    a.t[i].scales = reinterpret_cast<uint16_t *>(jobs[i].scales);
    a.t[i].gscale = jobs[i].gscale;
    a.t[i].partials = jobs[i].partials;
    a.t[i].units = jobs[i].rows * (jobs[i].cols / 32);
    a.t[i].units_per_row = (uint32_t)(jobs[i].cols / 32);
    a.t[i].ld = jobs[i].ld;
    if (a.t[i].units > max_units) max_units = a.t[i].units;
  }
  // Both tensors of a pair use the same grid; a tensor with fewer units simply
  // leaves some threads idle.
  const int nparts = amax_blocks(max_units);
  hipLaunchKernelGGL(k_amax, dim3(nparts, njobs), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_encode, dim3(encode_blocks(max_units), njobs), dim3(kThreads), 0, stream, a,
                     nparts);
  return hipGetLastError();
}

}  // namespace nvfp4
