// W4A4 NVFP4 GEMM for gfx950: C = bf16(Dequant(A) · Dequant(W)ᵀ · … ).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 量化格式
// (Dequant = X^FP4 · α^FP8 · α^FP32) and 推理底座 (W4A4 inference: weights
// materialised once in 4 bits, activations quantised per call).  Reductions in
// higher precision (二、方法 / NVFP4 训练的工程细节): FP32 accumulation, FP32
// epilogue.
//
// How the 16-wide E4M3 block scales meet the matrix cores.  gfx950's scaled
// MFMA takes one power-of-two (E8M0) scale per 32 elements, and its fp4
// converters apply only the exponent of their scale operand, so neither can
// carry an NVFP4 scale exactly.  An element times its block scale, E2M1 · E4M3,
// has at most 6 significant bits and lies in [2^-10, 2688]: it is exact in
// fp16.  So each fragment is decoded exactly:
//   v_cvt_scalef32_pk_f16_fp4(codes, 2^8)  → E2M1 · 2^8            (exact)
//   v_pk_mul_f16(·, S · 2^-8)              → E2M1 · S              (exact)
// where the f16 pattern of S·2^-8 is just the E4M3 byte shifted left by 7
// (E4M3 and fp16 differ only in exponent bias, 7 vs 15, for normals and
// subnormals alike).  The fragments feed v_mfma_f32_32x32x16_f16; each
// product of two fragments is exact in fp32 and the sums accumulate in fp32.
// The epilogue applies fl32(Ag·Wg), the bias and optional GELU, and rounds to
// bf16 once.
//
// Tiling: 4 waves as 2 x 2; each wave owns (32·WM) activation rows x (32·WN)
// weight rows and keeps WM·WN 32x32 fp32 accumulators.  K advances in stages of
// 128 elements (64 code bytes + 8 scale bytes per row) through a
// double-buffered LDS ring.  Inside a stage each lane reads 16 code bytes of one
// row (32 consecutive k), i.e. four MFMA fragments; lanes 0-31 and 32-63 take
// adjacent 32-k halves.  That is a fixed permutation of k applied identically
// to both operands, which leaves the sum unchanged.  Code chunks sit in LDS
// chunk-major ([chunk][row][16 B], rows padded by 16) so the 16-byte reads of
// 32 consecutive rows are contiguous and the row-fastest fills are
// conflict-free.
#include <nvfp4.h>

#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kGemmThreads = 256;
constexpr int kBK = 128;                 // K elements per stage
constexpr int kChunks = kBK / 32;        // 16-byte code chunks per row per stage
constexpr int kPadRows = 16;

template <int WM, int WN>
struct Tile {
  static constexpr int BM = 64 * WM;
  static constexpr int BN = 64 * WN;
  static constexpr int A_CODE = 0;
  static constexpr int W_CODE = A_CODE + kChunks * (BM + kPadRows) * 16;
  static constexpr int A_SCALE = W_CODE + kChunks * (BN + kPadRows) * 16;
  static constexpr int W_SCALE = A_SCALE + BM * 8;
  static constexpr int STAGE = W_SCALE + BN * 8;
  static constexpr int LDS = 2 * STAGE;
};

// ---------------------------------------------------------------------------
// global → registers → LDS staging of one operand (ROWS rows) for one stage

template <int ROWS>
struct StageRegs {
  static constexpr int NC = ROWS * kChunks / kGemmThreads;   // code chunks per thread
  u32x4 code[NC];
  u32x2 scale;
};

template <int ROWS>
__device__ __forceinline__ void load_stage(StageRegs<ROWS> &s, const uint8_t *codes,
                                           const uint8_t *scales, int64_t row0, int64_t nrows,
                                           int64_t K, int ks, bool scale_aligned) {
  const int t = threadIdx.x;
  const int64_t row_bytes = K / 2;
  const int64_t col0 = (int64_t)ks * (kBK / 2);
#pragma unroll
  for (int it = 0; it < StageRegs<ROWS>::NC; ++it) {
    const int q = t + kGemmThreads * it;
    const int row = q % ROWS, c = q / ROWS;
    int64_t gr = row0 + row;
    gr = gr < nrows ? gr : nrows - 1;
    const int64_t col = col0 + 16 * c;
    if (col < row_bytes)
      s.code[it] = *reinterpret_cast<const u32x4 *>(codes + gr * row_bytes + col);
    else
      s.code[it] = u32x4{0u, 0u, 0u, 0u};
  }
  s.scale = u32x2{0u, 0u};
  if (t < ROWS) {
    int64_t gr = row0 + t;
    gr = gr < nrows ? gr : nrows - 1;
    const int64_t srow = K / 16;
    const int64_t scol = (int64_t)ks * (kBK / 16);
    const uint8_t *p = scales + gr * srow + scol;
    if (scale_aligned && scol + 8 <= srow) {
      s.scale = *reinterpret_cast<const u32x2 *>(p);
    } else {
      // unaligned row starts or a partial last stage: 2-byte pieces, masked
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (scol + 2 * b + 2 <= srow) w[b] = *reinterpret_cast<const uint16_t *>(p + 2 * b);
      s.scale = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
    }
  }
}

template <int ROWS>
__device__ __forceinline__ void store_stage(const StageRegs<ROWS> &s, uint8_t *code_lds,
                                            uint8_t *scale_lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < StageRegs<ROWS>::NC; ++it) {
    const int q = t + kGemmThreads * it;
    const int row = q % ROWS, c = q / ROWS;
    *reinterpret_cast<u32x4 *>(code_lds + (c * (ROWS + kPadRows) + row) * 16) = s.code[it];
  }
  if (t < ROWS) *reinterpret_cast<u32x2 *>(scale_lds + t * 8) = s.scale;
}

// ---------------------------------------------------------------------------
// fragment decode: 8 E2M1 codes (one dword) times one E4M3 block scale → f16x8

template <int SEL>
__device__ __forceinline__ f16x2 cvt2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, SEL);   // E2M1 · 2^8
}

__device__ __forceinline__ f16x8 decode8(uint32_t w, uint32_t scale_pair) {
  const f16x2 s = __builtin_bit_cast(f16x2, scale_pair);               // (S·2^-8, S·2^-8)
  const f16x2 p0 = cvt2<0>(w) * s, p1 = cvt2<1>(w) * s;
  const f16x2 p2 = cvt2<2>(w) * s, p3 = cvt2<3>(w) * s;
  const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E4M3 byte → the fp16 pattern of S·2^-8 in both halves.
__device__ __forceinline__ uint32_t scale_pair_f16(uint32_t byte) {
  return (byte & 0xFFu) * 0x00800080u;
}

// ---------------------------------------------------------------------------

__device__ __forceinline__ float gelu_tanh(float y) {
  // 0.5·y·(1 + tanh(z)) = y / (1 + e^(-2z)),  z = √(2/π)·(y + 0.044715·y³)
  const float z = 0.7978845608028654f * (y + 0.044715f * y * y * y);
  return y / (1.0f + __expf(-2.0f * z));
}

template <int WM, int WN>
__global__ void __launch_bounds__(kGemmThreads, 1) k_gemm(GemmArgs a, int tiles_m, int tiles_n) {
  using T = Tile<WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];

  // tile order: contiguous runs of tiles per XCD (workgroups are dealt to the
  // 8 XCDs round-robin), M-fastest inside groups of 8 M-tiles so concurrently
  // running tiles share weight rows in L2.
  int b = blockIdx.x;
  const int ntiles = tiles_m * tiles_n;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int grp = b / per_group, first_m = grp * GM;
  const int gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in = b - grp * per_group;
  const int tile_m = first_m + in % gsz, tile_n = in / gsz;

  const int64_t m0 = (int64_t)tile_m * T::BM, n0 = (int64_t)tile_n * T::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 31, h = lane >> 5;
  const int nk = (int)((a.K + kBK - 1) / kBK);
  const bool scale_aligned = (a.K % kBK) == 0;

  f32x16 acc[WN][WM];
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

  StageRegs<T::BM> ra;
  StageRegs<T::BN> rw;
  load_stage<T::BM>(ra, a.Aq, a.As, m0, a.M, a.K, 0, scale_aligned);
  load_stage<T::BN>(rw, a.Wq, a.Ws, n0, a.N, a.K, 0, scale_aligned);
  store_stage<T::BM>(ra, smem + T::A_CODE, smem + T::A_SCALE);
  store_stage<T::BN>(rw, smem + T::W_CODE, smem + T::W_SCALE);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    uint8_t *cur = smem + (ks & 1) * T::STAGE;
    uint8_t *nxt = smem + ((ks + 1) & 1) * T::STAGE;
    const bool more = ks + 1 < nk;
    if (more) {
      load_stage<T::BM>(ra, a.Aq, a.As, m0, a.M, a.K, ks + 1, scale_aligned);
      load_stage<T::BN>(rw, a.Wq, a.Ws, n0, a.N, a.K, ks + 1, scale_aligned);
    }

    u32x2 sa[WM], sw[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
      sa[i] = *reinterpret_cast<const u32x2 *>(cur + T::A_SCALE + (wm * 32 * WM + 32 * i + r) * 8);
#pragma unroll
    for (int j = 0; j < WN; ++j)
      sw[j] = *reinterpret_cast<const u32x2 *>(cur + T::W_SCALE + (wn * 32 * WN + 32 * j + r) * 8);

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 2 * s + h;
      u32x4 qa[WM], qw[WN];
      uint32_t sca[WM][2], scw[WN][2];
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        qa[i] = *reinterpret_cast<const u32x4 *>(
            cur + T::A_CODE + (c * (T::BM + kPadRows) + wm * 32 * WM + 32 * i + r) * 16);
        const uint32_t p = (s ? sa[i].y : sa[i].x) >> (16 * h);
        sca[i][0] = scale_pair_f16(p);
        sca[i][1] = scale_pair_f16(p >> 8);
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        qw[j] = *reinterpret_cast<const u32x4 *>(
            cur + T::W_CODE + (c * (T::BN + kPadRows) + wn * 32 * WN + 32 * j + r) * 16);
        const uint32_t p = (s ? sw[j].y : sw[j].x) >> (16 * h);
        scw[j][0] = scale_pair_f16(p);
        scw[j][1] = scale_pair_f16(p >> 8);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f16x8 fa[WM], fw[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i) fa[i] = decode8(qa[i][t], sca[i][t >> 1]);
#pragma unroll
        for (int j = 0; j < WN; ++j) fw[j] = decode8(qw[j][t], scw[j][t >> 1]);
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
          for (int i = 0; i < WM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fw[j], fa[i], acc[j][i], 0, 0, 0);
      }
    }

    if (more) {
      store_stage<T::BM>(ra, nxt + T::A_CODE, nxt + T::A_SCALE);
      store_stage<T::BN>(rw, nxt + T::W_CODE, nxt + T::W_SCALE);
    }
    __syncthreads();
  }

  // ---- epilogue: acc[j][i][v] is C[m][n] with m = (row block i) + r,
  //      n = (column block j) + 8·(v/4) + 4·h + v%4.  Each operation rounds
  //      on its own (no fused multiply-add), as the interface states.
  {
#pragma clang fp contract(off)
  const float gg = a.Ag[0] * a.Wg[0];
  const bool gelu = (a.flags & NVFP4_EPI_GELU_TANH) != 0;
  const bool vec_ok = (a.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < WN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = n0 + wn * 32 * WN + 32 * j + 8 * q + 4 * h;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.bias) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (n + k < a.N) bv[k] = bf16_bits_to_f32(a.bias[n + k]);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const int64_t m = m0 + wm * 32 * WM + 32 * i + r;
        float o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float y = acc[j][i][4 * q + k] * gg;
          if (a.bias) y = y + bv[k];
          if (gelu) y = gelu_tanh(y);
          o[k] = y;
        }
        if (m < a.M) {
          uint16_t *dst = a.C + m * a.N + n;
          if (vec_ok && n + 3 < a.N) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (n + k < a.N) dst[k] = (uint16_t)(pack_bf16x2(o[k], 0.0f) & 0xFFFFu);
          }
        }
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------

struct TileChoice {
  int wm, wn;
};

static TileChoice choose_tile(int64_t M, int64_t N) {
  // Pick the tile with the least estimated time: rounds of 256 concurrently
  // resident workgroups (one per CU) x per-tile cost, where a tile costs its
  // area plus a decode overhead that grows as the wave tile shrinks.
  const TileChoice cands[] = {{4, 4}, {4, 3}, {3, 4}, {4, 2}, {2, 4}, {2, 2}};
  TileChoice best = cands[0];
  double best_cost = 1e300;
  for (const TileChoice &c : cands) {
    const int64_t bm = 64 * c.wm, bn = 64 * c.wn;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t rounds = (tiles + 255) / 256;
    const double per_tile = (double)bm * bn * (1.0 + 0.25 * (1.0 / c.wm + 1.0 / c.wn));
    const double cost = rounds * per_tile;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

void gemm_tile_for(int64_t M, int64_t N, int64_t, int *bm, int *bn) {
  const TileChoice c = choose_tile(M, N);
  *bm = 64 * c.wm;
  *bn = 64 * c.wn;
}

template <int WM, int WN>
static hipError_t launch_t(const GemmArgs &a, hipStream_t stream) {
  using T = Tile<WM, WN>;
  const int tm = (int)((a.M + T::BM - 1) / T::BM), tn = (int)((a.N + T::BN - 1) / T::BN);
  hipLaunchKernelGGL((k_gemm<WM, WN>), dim3(tm * tn), dim3(kGemmThreads), 0, stream, a, tm, tn);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  static const TileChoice by_flag[] = {{0, 0}, {4, 4}, {4, 3}, {3, 4}, {4, 2}, {2, 4}, {2, 2}};
  const uint32_t tf = (a.flags & NVFP4_TILE_MASK) >> 8;
  const TileChoice c = tf ? by_flag[tf] : choose_tile(a.M, a.N);
  if (c.wm == 4 && c.wn == 4) return launch_t<4, 4>(a, stream);
  if (c.wm == 4 && c.wn == 3) return launch_t<4, 3>(a, stream);
  if (c.wm == 3 && c.wn == 4) return launch_t<3, 4>(a, stream);
  if (c.wm == 4 && c.wn == 2) return launch_t<4, 2>(a, stream);
  if (c.wm == 2 && c.wn == 4) return launch_t<2, 4>(a, stream);
  return launch_t<2, 2>(a, stream);
}

}  // namespace nvfp4
