// Random Hadamard transform of a weight-gradient operand and NVFP4
// quantisation of its transpose (gfx950).
//
// Source: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 训练的工程细节
// (the operands of the weight-gradient GEMM pass through a random Hadamard
// transform before they are quantised; gradients take 1-D block scales) and
// 二、方法 / NVFP4 量化格式 (E2M1 elements, E4M3 scale per 16, FP32 tensor scale).
//
// dW[o, i] = Σ_t dy[t, o]·x[t, i] contracts over tokens, and the GEMM takes
// each operand with the contraction axis contiguous.  So an operand x [T, N]
// (tokens × features, row-major) is transformed along T and written as its
// transpose: codes [N, T/2], scales [N, T/16].  Per group of 16 tokens,
// y = H16·diag(s)·x/4 (Sylvester's H16, s_k = −1 where bit k of the mask is
// set); using the same signs on both operands leaves the product unchanged.
//
// Arithmetic.  The butterflies run in binary64, where a sum of 16 bf16 values
// is exact unless the group spans 2^41 or more in magnitude; each output is
// rounded once to binary32 (an exact zero as +0: a sign-flipped zero input
// would otherwise leave −0 in the sums).  The factor 1/4 is a power of two,
// so the kernel keeps u = fl32(4y) and applies 1/4 exactly where y enters:
// the block amax (a = max|u| / 4) and the reciprocal (u·(r/4) rounds like
// y·r).  The tensor amax, the E4M3 block scales and the E2M1 codes then follow
// the binary32 steps of the NVFP4 quantiser.
//
// Layout of the work.  A workgroup pass covers 256 tokens × 16·kFeat
// features with 256 threads; thread (group = tid/16, c = tid%16) holds the 16
// tokens of one group for kFeat consecutive features (16 loads of 2·kFeat
// bytes: one wave reads four row segments of 32·kFeat bytes per load).  Each
// of its columns is exactly one NVFP4 block of the transpose, so block maxima
// need no exchange between threads.  kFeat = 4 keeps the encode kernel at
// three waves per SIMD (8 features need two and were 7 % slower on an
// 8192 × 14336 operand; prefetching the next tile into registers cost more
// occupancy than it hid).  The code bytes (128 per feature) and scale bytes
// (16 per feature) of the transpose are staged in LDS and written as whole
// row segments.
//
// Two launches, because the tensor amax of the transformed values precedes
// every block scale: the first writes one partial amax per workgroup; the
// second folds them into g, then transforms again and encodes, visiting the
// tiles in reverse order (the first launch's last tiles first).
#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kFeat = 4;                     // features per thread (one 8-byte load per token)
constexpr int kWords = kFeat / 2;            // bf16 pairs per token and thread
constexpr int kTileT = 256;                  // tokens per workgroup pass
constexpr int kTileN = 16 * kFeat;           // features per workgroup pass
constexpr int kCodeStride = kTileT / 2 + 16; // LDS row of code bytes, 16-byte aligned
typedef __attribute__((ext_vector_type(kWords))) uint32_t load_t;

struct Tile {
  int64_t t0, n0;
};

__device__ __forceinline__ Tile tile_of(const RhtArgs &a, int64_t tile) {
  const int64_t ntn = (a.N + kTileN - 1) / kTileN;
  return Tile{(tile / ntn) * kTileT, (tile % ntn) * kTileN};
}

// The 16 tokens of this thread's group × its kFeat features, as bf16 pairs
// (w[i][d] holds features 2d, 2d+1 of token i), each row's sign applied.
// Tokens past T and features past N read as 0.
__device__ __forceinline__ void load_group(const RhtArgs &a, const Tile &tl, uint32_t (&w)[16][kWords]) {
  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int64_t t = tl.t0 + 16 * grp, n = tl.n0 + kFeat * c;
  if (t >= a.T || n >= a.N) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int d = 0; d < kWords; ++d) w[i][d] = 0u;
    return;
  }
  const uint16_t *p = a.x + t * a.ld + n;
  if (n + kFeat <= a.N) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const load_t v = *reinterpret_cast<const load_t *>(p + i * a.ld);
#pragma unroll
      for (int d = 0; d < kWords; ++d) w[i][d] = v[d];
    }
  } else {
    const int valid = (int)(a.N - n);
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int d = 0; d < kWords; ++d) {
        const uint32_t lo = (2 * d < valid) ? p[i * a.ld + 2 * d] : 0u;
        const uint32_t hi = (2 * d + 1 < valid) ? p[i * a.ld + 2 * d + 1] : 0u;
        w[i][d] = lo | (hi << 16);
      }
  }
  // s_i applies to every feature of token i: flip both bf16 signs of a pair
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t flip = ((a.sign_mask >> i) & 1u) ? 0x80008000u : 0u;
#pragma unroll
    for (int d = 0; d < kWords; ++d) w[i][d] ^= flip;
  }
}

// v ← H16·v in Sylvester order (H[i, k] = (−1)^popcount(i & k)), binary64:
// four radix-2 stages of sums and differences.
__device__ __forceinline__ void fwht16(double (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const double p = v[i], q = v[i + h];
        v[i] = p + q;
        v[i + h] = p - q;
      }
}

// Feature e of the thread's group, signed, as binary64, transformed.
__device__ __forceinline__ void column(const uint32_t (&w)[16][kWords], int e, double (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t d = w[i][e >> 1];
    v[i] = (double)__uint_as_float((e & 1) ? (d & 0xFFFF0000u) : (d << 16));
  }
  fwht16(v);
}

__global__ void __launch_bounds__(kThreads) k_rht_amax(RhtArgs a, int64_t ntiles) {
  double m = 0.0;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    uint32_t w[16][kWords];
    load_group(a, tile_of(a, tile), w);
#pragma unroll
    for (int e = 0; e < kFeat; ++e) {
      double v[16];
      column(w, e, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = __builtin_fmax(m, __builtin_fabs(v[i]));
    }
  }
  // max |fl32(v)| = fl32(max |v|) (rounding is monotone); y = fl32(v)/4 exactly
  uint32_t mu = __float_as_uint((float)m * 0.25f);
  mu = wave_max_u32(mu);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mu;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) r = r > red[i] ? r : red[i];
    a.partials[blockIdx.x] = r;
  }
}

// Codes of the pair (u0, u1) scaled by r, into byte SEL of old.  The converter
// rounds to nearest even, saturates at ±6 and keeps the sign of zero.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pair_f32(uint32_t old, float u0, float u1, float r) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, u0 * r, u1 * r, 1.0f, SEL);
}

__global__ void __launch_bounds__(kThreads) k_rht_encode(RhtArgs a, int64_t ntiles, int nparts) {
  __shared__ __attribute__((aligned(16))) uint8_t cd[kTileN * kCodeStride];
  __shared__ __attribute__((aligned(16))) uint8_t sc[kTileN * 16];
  __shared__ uint32_t red[kThreads / 64];

  // g from the partial maxima (binary32 magnitudes, so their bit patterns order like them)
  uint32_t mu = 0;
  for (int p = threadIdx.x; p < nparts; p += kThreads) {
    const uint32_t v = a.partials[p];
    mu = mu > v ? mu : v;
  }
  mu = wave_max_u32(mu);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mu;
  __syncthreads();
  uint32_t A = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) A = A > red[i] ? A : red[i];
  const float g = (A == 0) ? 1.0f : __uint_as_float(A) / kGlobalDivisor;   // fl(A / 2688)
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.gscale = g;
  const BlockScaler b6(g, kE2M1Max);

  const int grp = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int64_t half_t = a.T / 2, sixteenth_t = a.T / 16;
  for (int64_t tile = ntiles - 1 - blockIdx.x; tile >= 0; tile -= gridDim.x) {
    const Tile tl = tile_of(a, tile);
    uint32_t w[16][kWords];
    load_group(a, tl, w);
#pragma unroll
    for (int e = 0; e < kFeat; ++e) {
      double v[16];
      column(w, e, v);
      float u[16];
      float au = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        u[i] = (float)v[i] + 0.0f;                            // fl32(4y), an exact zero as +0
        au = __builtin_fmaxf(au, __builtin_fabsf(u[i]));
      }
      const uint32_t S = b6.scale_byte_of(au * 0.25f);         // block amax of y
      const float r = b6.recip(S) * 0.25f;                     // u·r/4 rounds like y·r
      uint32_t lo = 0, hi = 0;
      lo = cvt_pair_f32<0>(lo, u[0], u[1], r);
      lo = cvt_pair_f32<1>(lo, u[2], u[3], r);
      lo = cvt_pair_f32<2>(lo, u[4], u[5], r);
      lo = cvt_pair_f32<3>(lo, u[6], u[7], r);
      hi = cvt_pair_f32<0>(hi, u[8], u[9], r);
      hi = cvt_pair_f32<1>(hi, u[10], u[11], r);
      hi = cvt_pair_f32<2>(hi, u[12], u[13], r);
      hi = cvt_pair_f32<3>(hi, u[14], u[15], r);
      const int row = kFeat * c + e;                           // feature within the tile
      *reinterpret_cast<u32x2 *>(cd + row * kCodeStride + 8 * grp) = u32x2{lo, hi};
      sc[row * 16 + grp] = (uint8_t)S;
    }
    __syncthreads();
    // kTileN rows × 8 chunks of 16 code bytes (32 tokens each); T is a
    // multiple of 32, so a chunk is wholly inside or outside the tensor
#pragma unroll
    for (int it = 0; it < kTileN * 8 / kThreads; ++it) {
      const int q = threadIdx.x + kThreads * it;
      const int row = q >> 3, part = q & 7;
      const int64_t n = tl.n0 + row;
      if (n < a.N && tl.t0 + 32 * part < a.T) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(cd + row * kCodeStride + 16 * part);
        *reinterpret_cast<u32x4 *>(a.codes + n * half_t + tl.t0 / 2 + 16 * part) = v;
      }
    }
    // kTileN rows × 8 pairs of scale bytes (32 tokens each)
#pragma unroll
    for (int it = 0; it < kTileN * 8 / kThreads; ++it) {
      const int q = threadIdx.x + kThreads * it;
      const int row = q >> 3, pr = q & 7;
      const int64_t n = tl.n0 + row;
      if (n < a.N && tl.t0 + 32 * pr < a.T) {
        const uint16_t v = *reinterpret_cast<const uint16_t *>(sc + row * 16 + 2 * pr);
        *reinterpret_cast<uint16_t *>(a.scales + n * sixteenth_t + tl.t0 / 16 + 2 * pr) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

int64_t rht_tiles(int64_t T, int64_t N) {
  return ((T + kTileT - 1) / kTileT) * ((N + kTileN - 1) / kTileN);
}

hipError_t launch_quantize_rht(const RhtArgs &a, hipStream_t stream) {
  const int64_t ntiles = rht_tiles(a.T, a.N);
  const int grid = (int)(ntiles < kRhtMaxParts ? ntiles : kRhtMaxParts);
  hipLaunchKernelGGL(k_rht_amax, dim3(grid), dim3(kThreads), 0, stream, a, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rht_encode, dim3(grid), dim3(kThreads), 0, stream, a, ntiles, grid);
  return hipGetLastError();
}

}  // namespace nvfp4
