// K-smoothing of an appended KV chunk (gfx950): the per-channel centre of the
// chunk's keys and the smoothed keys that are then quantised.
//
// Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座 (each
// KV chunk is quantised again on its own, with K-smoothing on its keys).  The
// pages name K-smoothing without defining it; the definition used here:
//   centre of channel c over the chunk's T tokens
//     z_t = clamp(round_half_even(K[t, c] · 2^24), −2^38, 2^38)
//     S   = Σ_t z_t                     (exact, 64-bit integers, any order)
//     μ_c = bf16_rne(fl64(fl64(S) / T) · 2^-24)
//   smoothed key K'[t, c] = bf16_rne(fl32(K[t, c] − μ_c)), formed by the
//   quantiser as it loads each block of K (the append passes it the centres).
// Because the sum is exact integer arithmetic, the centre does not depend on
// the order in which the parts are added.  The workspace needs no
// initialisation: every partial sum is written before it is read.
//
// Short chunks (at most kDirectMaxT tokens: one frame, the tail of a
// sequence) take one launch before the append's quantiser:
//   k_kv_center_direct — 16 channels per 1024-thread workgroup: every lane
//                  sums 8 channels over every 512th token (exact binary64),
//                  the 512 token rows meet in LDS as 64-bit integers, and
//                  one thread per channel turns the sum into μ.
// Longer chunks take two:
//   k_kv_colsum  — workgroups own a strip of tokens (sized so that about 1024
//                  workgroups cover the chunk) x 512 channels; every lane sums
//                  8 channels over every fourth token of the strip (16-byte
//                  loads along the channels, four in flight; grid steps in
//                  binary32, lane sums in exact binary64), the four token
//                  rows of a workgroup meet in LDS, and the workgroup stores
//                  its partial sum of each channel;
//   k_kv_center  — 64 channels per workgroup: its four waves add every
//                  fourth strip's partial sums, meet in LDS, and one thread
//                  per channel turns the sum into μ and writes it to the
//                  cache's centre row of this append.
// The quantiser then reads K once more, centres each block as it loads it,
// and encodes K' (and V) as for an unsmoothed append.
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kSmThreads = 256;
constexpr int kSmChan = 512;              // channels per colsum workgroup (64 lanes x 8)
constexpr int kSmRows = kSmThreads / 64;  // token rows per colsum workgroup
constexpr int kSmUnroll = 4;              // loads of a lane in flight together
constexpr int kSmTargetWgs = 1024;        // colsum workgroups aimed at (four per CU)
constexpr int kDirThreads = 1024;         // k_kv_center_direct: 2 lanes x 8 channels x 512 token rows
constexpr int kDirChan = 16;              // channels per k_kv_center_direct workgroup
constexpr int kDirRows = kDirThreads / (kDirChan / 8);
constexpr int64_t kDirectMaxT = 2304;     // longest chunk summed by k_kv_center_direct

// Tokens per colsum strip: a multiple of 16 (4 rows x 4 loads in flight),
// long enough that about kSmTargetWgs workgroups cover the chunk.
static int64_t smooth_strip(int64_t T, int64_t e) {
  const int64_t cgroups = (e + kSmChan - 1) / kSmChan;
  int64_t strip = (T * cgroups + kSmTargetWgs - 1) / kSmTargetWgs;
  strip = (strip + kSmRows * kSmUnroll - 1) / (kSmRows * kSmUnroll) * (kSmRows * kSmUnroll);
  strip = strip > (int64_t(1) << 17) ? (int64_t(1) << 17) : strip;   // exact binary64 lane sums
  return strip < kSmRows * kSmUnroll ? kSmRows * kSmUnroll : strip;
}

// The key's count of 2^-24 steps, nearest-even, saturated at ±2^38, in
// binary32 without branches: K·2^24 is exact (8 significant bits; keys beyond
// 2^104 become infinite and saturate), round-to-nearest-even to an integer is
// exact, and so is the saturation at ±2^38.  The lanes add these counts in
// binary64, exact while a lane adds at most 2^15 of them (strips are capped at
// 2^17 tokens: 4 rows of 2^15), and convert to 64-bit integers once.
__device__ __forceinline__ float grid_steps_f32(uint32_t bf16) {
  float x = __builtin_rintf(bf16_bits_to_f32(bf16) * 16777216.0f);
  x = __builtin_fmaxf(x, -274877906944.0f);
  return __builtin_fminf(x, 274877906944.0f);
}

__global__ void __launch_bounds__(kSmThreads) k_kv_colsum(SmoothArgs a, int64_t strip) {
  __shared__ int64_t red[kSmRows][64][8];
  const int lane = threadIdx.x & 63, row = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.y * kSmChan + 8 * lane;
  const int64_t t0 = (int64_t)blockIdx.x * strip + row;
  int64_t t1 = t0 - row + strip;
  t1 = t1 < a.T ? t1 : a.T;
  double accd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < a.e) {
    for (int64_t tb = t0; tb < t1; tb += kSmRows * kSmUnroll) {
      u32x4 v[kSmUnroll];
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) {
        const int64_t t = tb + (int64_t)kSmRows * i;
        v[i] = t < t1 ? *reinterpret_cast<const u32x4 *>(a.k + t * a.ld + c0) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          accd[2 * k] += (double)grid_steps_f32(w[k] & 0xFFFFu);   // +0 steps for the padding zeros
          accd[2 * k + 1] += (double)grid_steps_f32(w[k] >> 16);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[row][lane][k] = (int64_t)accd[k];
  __syncthreads();
  // thread j adds channels 2j and 2j + 1 of the workgroup's 512 and stores
  // the strip's partial sums
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ch = 2 * threadIdx.x + h;
    const int64_t c = (int64_t)blockIdx.y * kSmChan + ch;
    if (c < a.e) {
      int64_t s = 0;
#pragma unroll
      for (int r = 0; r < kSmRows; ++r) s += red[r][ch >> 3][ch & 7];
      a.partials[(int64_t)blockIdx.x * a.e + c] = s;
    }
  }
}

// Nearest-even bf16 of a binary64 value in the centre's range: 0 or a
// magnitude in [2^-48, 2^14] (a normal bf16): 7 of the 52 fraction bits kept.
__device__ __forceinline__ uint16_t bf16_rne_from_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t sign = (uint32_t)(b >> 63) << 15;
  const uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return (uint16_t)sign;
  uint32_t exp = (uint32_t)(mag >> 52) - 1023u + 127u;
  uint64_t keep = (mag & 0xFFFFFFFFFFFFFull) >> 45;
  const uint64_t rem = mag & ((uint64_t(1) << 45) - 1), half = uint64_t(1) << 44;
  if (rem > half || (rem == half && (keep & 1u))) ++keep;
  if (keep == 128) {
    keep = 0;
    ++exp;
  }
  return (uint16_t)(sign | (exp << 7) | (uint32_t)keep);
}

// Workgroups own 64 channels; the four waves add every fourth strip's
// partial sums and meet in LDS.
__global__ void __launch_bounds__(kSmThreads) k_kv_center(SmoothArgs a, int64_t strips) {
  __shared__ int64_t red[kSmRows][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  int64_t S = 0;                                   // exact: |S| <= 2^62
  if (c < a.e) {
    int64_t p = w;
    for (; p + kSmRows * (kSmUnroll - 1) < strips; p += kSmRows * kSmUnroll) {
      int64_t v[kSmUnroll];
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) v[i] = a.partials[(p + kSmRows * i) * a.e + c];
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) S += v[i];
    }
    for (; p < strips; p += kSmRows) S += a.partials[p * a.e + c];
  }
  red[w][lane] = S;
  __syncthreads();
  if (w != 0 || c >= a.e) return;
  S = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  const double mean = (double)S / (double)a.T;
  a.center[c] = bf16_rne_from_f64(mean * 0x1p-24);
}

// Sum and centre in one launch for a short chunk: channel group x (16
// channels, 16x .. 16x+15) goes to workgroup 8·(x mod n/8) + x div (n/8)
// when the n groups split evenly over the 8 XCDs (workgroup w runs on XCD
// w mod 8), so the four groups that share a 128-byte line of a token row are
// read on one XCD and its L2 fetches the line once; thread (row = t/2, octet o = t%2) adds channels 16x+8o .. +7
// of tokens row, row + 512, ... in binary64 (at most 5 values of magnitude
// <= 2^38 per lane: exact), then the rows meet in LDS as 64-bit integers.
__global__ void __launch_bounds__(kDirThreads) k_kv_center_direct(SmoothArgs a) {
  __shared__ int64_t red[kDirRows][kDirChan];
  __shared__ int64_t red2[32][kDirChan];
  const int oct = threadIdx.x % (kDirChan / 8), row = threadIdx.x / (kDirChan / 8);
  const int64_t n = gridDim.x, w = blockIdx.x;
  const int64_t grp = (n % 8 == 0) ? (w % 8) * (n / 8) + w / 8 : w;
  const int64_t c0 = grp * kDirChan + 8 * oct;
  double accd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < a.e) {
    for (int64_t tb = row; tb < a.T; tb += (int64_t)kDirRows * kSmUnroll) {
      u32x4 v[kSmUnroll];
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) {
        const int64_t t = tb + (int64_t)kDirRows * i;
        v[i] = t < a.T ? *reinterpret_cast<const u32x4 *>(a.k + t * a.ld + c0) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kSmUnroll; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          accd[2 * k] += (double)grid_steps_f32(w[k] & 0xFFFFu);   // +0 steps for the padding zeros
          accd[2 * k + 1] += (double)grid_steps_f32(w[k] >> 16);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[row][8 * oct + k] = (int64_t)accd[k];
  __syncthreads();
  if (threadIdx.x < 32 * kDirChan) {       // 32 parts of kDirRows/32 rows per channel
    const int c = threadIdx.x % kDirChan, part = threadIdx.x / kDirChan;
    int64_t S = 0;
#pragma unroll
    for (int r = 0; r < kDirRows / 32; ++r) S += red[part * (kDirRows / 32) + r][c];
    red2[part][c] = S;
  }
  __syncthreads();
  const int64_t c = grp * kDirChan + threadIdx.x;
  if (threadIdx.x >= kDirChan || c >= a.e) return;
  int64_t S = 0;                           // exact: |S| <= 2^38 · 2304
#pragma unroll
  for (int p = 0; p < 32; ++p) S += red2[p][threadIdx.x];
  const double mean = (double)S / (double)a.T;
  a.center[c] = bf16_rne_from_f64(mean * 0x1p-24);
}

int64_t smooth_partial_count(int64_t T, int64_t e) {
  const int64_t strip = smooth_strip(T, e);
  return (T + strip - 1) / strip * e;
}

hipError_t launch_kv_smooth(const SmoothArgs &a, hipStream_t stream) {
  if (a.T < 1 || a.e < 8 || a.e % 8) return hipErrorInvalidValue;
  if (a.T <= kDirectMaxT) {
    const int64_t groups = (a.e + kDirChan - 1) / kDirChan;
    if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_kv_center_direct, dim3((unsigned)groups), dim3(kDirThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t strip = smooth_strip(a.T, a.e);
  const int64_t strips = (a.T + strip - 1) / strip, cgroups = (a.e + kSmChan - 1) / kSmChan;
  if (strips > 0x7FFFFFFF || cgroups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kv_colsum, dim3((unsigned)strips, (unsigned)cgroups), dim3(kSmThreads), 0, stream, a,
                     strip);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_kv_center, dim3((unsigned)((a.e + 63) / 64)), dim3(kSmThreads), 0, stream, a, strips);
  return hipGetLastError();
}

}  // namespace nvfp4
