// W4A4 NVFP4 GEMM kernel for gfx950: C = bf16(Dequant(A) · Dequant(W)ᵀ · … ).
// Each workgroup-tile shape is instantiated in a translation unit of its own
// (gemm_tile_<WM>x<WN>.hip, built in parallel); gemm.hip picks the tile.
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
// Tiling: 4 waves as 2 x 2, one wave per SIMD; each wave owns (32·WM)
// activation rows x (32·WN) weight rows and keeps WM·WN 32x32 fp32 accumulators
// (AGPRs).  K advances in stages of 128 elements (64 code bytes + 8 scale
// bytes per row in memory) through two LDS buffers: the workgroup copies stage ks+1 from
// registers into LDS and fetches stage ks+2 from L2 into registers while it
// computes stage ks.  Global loads move 64 contiguous bytes of a row per 4
// lanes (buffer loads; bytes past the tile read as 0); LDS holds codes
// chunk-major, [chunk][row + 4][16 B], so both the fills and the 16-byte
// fragment reads of 32 consecutive rows are free of bank conflicts.
// Lane (r, h) reads chunk 2s + h of row r in sub-step s: k = 64s + 32h + 8t + e
// for dword t, element e — a fixed permutation of k applied identically to
// both operands, which leaves the sum unchanged.  The block scales are stored
// in LDS already expanded to fp16 scale pairs (once per workgroup at fill
// time).  Decoding, not data movement, is the scarce resource (the fp16
// fragments' VALU work overlaps the MFMAs only in part): the decode of step
// t+1 is issued between the MFMAs of step t (explicit scheduling groups), and
// the first decode of the next stage overlaps the last MFMAs of the current
// one.
//
// Launch: one workgroup per CU loops over its tiles (persistent), fetching the
// next tile's first stage before the current epilogue; the 256x256 tile runs
// one tile per workgroup.  In the epilogue every lane stores 16 contiguous
// bytes of a row of C, gathered from the accumulator layout by a half-wave
// lane swap (v_permlane32_swap), with no LDS staging; tiles at the edges guard
// their stores per lane.  It can record the largest |output| of each tile (the
// linear layer's NVFP4 hand-off).
#pragma once

#include <nvfp4.h>

#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kGemmThreads = 256;
constexpr int kBK = 128;                 // K elements per stage

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
  // 0.5·y·(1 + tanh z) = y / (1 + e^(-2z)),  z = √(2/π)·(y + 0.044715·y³),
  // with e^(-2z) = 2^(y·(c1 + c2·y²)), c1 = -2·log2(e)·√(2/π), c2 = 0.044715·c1:
  // one exp2 and one reciprocal (each about 1 ulp), no division.  Large |y|
  // give y (exp2 → 0) or -0 (exp2 → inf, reciprocal → 0).
  constexpr float c1 = -2.302208198144325f, c2 = -0.1029432395800235f;
  const float t = y * (c1 + c2 * (y * y));
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

constexpr int kChunks = kBK / 32;        // 16-byte code chunks per row per stage
constexpr int kPadRows = 2;              // LDS row padding per chunk column
// rows of each operand's scale-pair region: one per thread, so every thread
// stores its own row (the rows past the tile's are never read)
constexpr int kScaleRows = kGemmThreads;

template <int WM, int WN>
struct Tile {
  static constexpr int BM = 64 * WM, BN = 64 * WN;
  static constexpr int A_CODE = 0;
  static constexpr int W_CODE = A_CODE + kChunks * (BM + kPadRows) * 16;
  static constexpr int A_SCALE = W_CODE + kChunks * (BN + kPadRows) * 16;   // [2][256][4 pairs]
  static constexpr int W_SCALE = A_SCALE + kScaleRows * 32;
  static constexpr int STAGE = W_SCALE + kScaleRows * 32;
  static constexpr int GG = 2 * STAGE;      // fl32(Ag·Wg)
  static constexpr int BIAS = GG + 16;      // [BN] bf16 bias of the tile's columns
  static constexpr int LDS = BIAS + BN * 2;
};

struct Operand {
  const uint8_t *codes;     // first row of the tile
  const uint8_t *scales;
  uint32_t code_bytes;      // bytes of the tile's rows (loads beyond read 0)
  uint32_t scale_bytes;
};

// One operand's share of a stage in flight in registers: ROWS·4 code chunks
// over 256 threads (4 lanes per row, 64 contiguous bytes), 8 scale bytes for
// the first ROWS threads.
template <int ROWS>
struct Fill {
  static constexpr int NC = ROWS * kChunks / kGemmThreads;
  u32x4 code[NC];
  u32x2 scale;
};

template <int ROWS, bool KTAIL>
__device__ __forceinline__ void fill_load(Fill<ROWS> &f, const Operand &op, int64_t K, int ks) {
  const int t = threadIdx.x;
  const uint32_t rb = (uint32_t)(K / 2), sb = (uint32_t)(K / 16);
  const uint32_t coff = (uint32_t)ks * (kBK / 2), soff = (uint32_t)ks * (kBK / 16);
  const uint32_t cn = op.code_bytes > coff ? op.code_bytes - coff : 0u;
  const uint32_t sn = op.scale_bytes > soff ? op.scale_bytes - soff : 0u;
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(op.codes + coff, cn);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(op.scales + soff, sn);
#pragma unroll
  for (int it = 0; it < Fill<ROWS>::NC; ++it) {
    const int q = t + kGemmThreads * it;
    const int row = q >> 2, c = q & 3;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(row * rb + 16 * c), 0, 0);
    f.code[it] = (KTAIL && coff + 16 * c >= rb) ? u32x4{0u, 0u, 0u, 0u} : v;
  }
  // threads past the last row reload (and later re-store) the last row: no
  // divergent branch in the main loop
  const int srow = t < ROWS ? t : ROWS - 1;
  if (!KTAIL) {
    f.scale = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(srow * sb), 0, 0);
  } else {   // scale rows only 2-byte aligned, last stage partial
    uint32_t w[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(srow * sb + 2 * b), 0, 0);
      w[b] = (soff + 2 * b >= sb) ? 0u : (v & 0xFFFFu);
    }
    f.scale = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
  }
}

// Codes go to LDS as they are; the 8 scale bytes of a row are expanded to
// fp16 scale pairs (scale_pair_f16) and stored as two 16-byte groups, blocks
// {0, 1, 4, 5} in the first kScaleRows·16 bytes and {2, 3, 6, 7} in the next: group
// h holds the blocks 2h, 2h+1, 4+2h, 5+2h that a lane with that h decodes, and
// a wave's accesses to one group are contiguous.
template <int ROWS>
__device__ __forceinline__ void fill_store(const Fill<ROWS> &f, uint8_t *code_lds, uint8_t *scale_lds) {
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Fill<ROWS>::NC; ++it) {
    const int q = t + kGemmThreads * it;
    const int row = q >> 2, c = q & 3;
    *reinterpret_cast<u32x4 *>(code_lds + (c * (ROWS + kPadRows) + row) * 16) = f.code[it];
  }
  // every thread stores its own row (threads past the tile's rows store a
  // copy of the last row that nothing reads), so no two lanes share an address
  const uint32_t lo = f.scale.x, hi = f.scale.y;     // blocks 0..3, 4..7
  const u32x4 g0 = {scale_pair_f16(lo), scale_pair_f16(lo >> 8), scale_pair_f16(hi), scale_pair_f16(hi >> 8)};
  const u32x4 g1 = {scale_pair_f16(lo >> 16), scale_pair_f16(lo >> 24), scale_pair_f16(hi >> 16),
                    scale_pair_f16(hi >> 24)};
  *reinterpret_cast<u32x4 *>(scale_lds + t * 16) = g0;
  *reinterpret_cast<u32x4 *>(scale_lds + (kScaleRows + t) * 16) = g1;
}

// A wave's view of one stage: codes of both sub-steps and the lane's four
// fp16 scale pairs, per row block q (A blocks first, then W blocks).
template <int NQ>
struct Frag {
  u32x4 c[2][NQ];
  u32x4 sc[NQ];
};

template <int WM, int WN>
__device__ __forceinline__ void frag_read(Frag<WM + WN> &fr, const uint8_t *buf, int wm, int wn,
                                          int r, int h) {
  using T = Tile<WM, WN>;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int row = wm * 32 * WM + 32 * i + r;
    fr.sc[i] = *reinterpret_cast<const u32x4 *>(buf + T::A_SCALE + (h * kScaleRows + row) * 16);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      fr.c[s][i] = *reinterpret_cast<const u32x4 *>(buf + T::A_CODE + ((2 * s + h) * (T::BM + kPadRows) + row) * 16);
  }
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int row = wn * 32 * WN + 32 * j + r;
    fr.sc[WM + j] = *reinterpret_cast<const u32x4 *>(buf + T::W_SCALE + (h * kScaleRows + row) * 16);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      fr.c[s][WM + j] = *reinterpret_cast<const u32x4 *>(buf + T::W_CODE + ((2 * s + h) * (T::BN + kPadRows) + row) * 16);
  }
}

// Decode step T (0..7) of a stage into fragments f: dword T%4 of sub-step T/4,
// block 4·(T/4) + 2h + (T%4)/2 of the stage → scale pair 2·(T/4) + (T%4)/2 of
// the lane's group.
template <int T, int NQ>
__device__ __forceinline__ void decode_step(const Frag<NQ> &fr, int, f16x8 (&f)[NQ]) {
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    f[q] = decode8(fr.c[T >> 2][q][T & 3], fr.sc[q][2 * (T >> 2) + ((T & 3) >> 1)]);
}

template <int WM, int WN>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[WN][WM], const f16x8 (&f)[WM + WN]) {
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
      acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f[WM + j], f[i], acc[j][i], 0, 0, 0);
}

// Scheduling groups for one step: one MFMA, then up to VPM VALU ops, repeated;
// in step 0 each of the first MFMAs also takes one LDS store of the fill, in
// step 1 one global load of the next fill.
template <int WM, int WN, int STEP>
__device__ __forceinline__ void interleave_hint() {
  constexpr int VPM = (9 * (WM + WN) + WM * WN - 1) / (WM * WN);
  constexpr int NFILL = WM + WN + 2;          // fill instructions per thread of each kind
#pragma unroll
  for (int k = 0; k < WM * WN; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    if (STEP == 0 && k < NFILL) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if (STEP == 1 && k < NFILL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// PERSIST: the workgroup loops over tiles w, w + grid, ... and prefetches the
// next tile's first stage under the current epilogue; otherwise one tile per
// workgroup (the 256x256 tile has no registers left for the loop state).
// GELU is a template parameter: a per-element test would leave a large,
// mostly skipped body in the epilogue, costing instruction fetches and a
// branch for every element.
template <int WM, int WN, bool KTAIL, bool PERSIST, bool GELU>
__global__ void __launch_bounds__(kGemmThreads, 1) k_gemm(GemmArgs a, int tiles_m, int tiles_n) {
  using T = Tile<WM, WN>;
  constexpr int BM = T::BM, BN = T::BN, NQ = WM + WN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];

  const int ntiles = tiles_m * tiles_n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 31, h = lane >> 5;
  const int nk = (int)((a.K + kBK - 1) / kBK);
  const int64_t rb = a.K / 2, sbytes = a.K / 16;

  // Tile t → (m0, n0): contiguous runs of tiles per XCD (workgroup w runs on
  // XCD w % 8 and processes tiles w, w + grid, ... with grid a multiple of 8,
  // so every tile it gets maps to its own XCD's run), M-fastest inside groups
  // of 8 M-tiles so concurrently running tiles share weight rows in L2.
  // Rows past the matrix end are outside the buffer ranges and read as 0;
  // their results are not stored.
  int64_t m0 = 0, n0 = 0;
  Operand opa, opw;
  auto setup = [&](int t) {
    int b = t;
    if ((ntiles & 7) == 0 && (gridDim.x & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int grp = b / per_group, first_m = grp * GM;
    const int gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
    const int in = b - grp * per_group;
    m0 = (int64_t)(first_m + in % gsz) * BM;
    n0 = (int64_t)(in / gsz) * BN;
    const int64_t rows_a = (a.M - m0) < BM ? (a.M - m0) : BM;
    const int64_t rows_w = (a.N - n0) < BN ? (a.N - n0) : BN;
    opa = Operand{a.Aq + m0 * rb, a.As + m0 * sbytes, (uint32_t)(rows_a * rb), (uint32_t)(rows_a * sbytes)};
    opw = Operand{a.Wq + n0 * rb, a.Ws + n0 * sbytes, (uint32_t)(rows_w * rb), (uint32_t)(rows_w * sbytes)};
  };

  f32x16 acc[WN][WM];
  Fill<BM> fa;
  Fill<BN> fw;
  Frag<NQ> fr;
  f16x8 f0[NQ], f1[NQ];

  // The epilogue's inputs, the bias of the tile's columns (one element per
  // thread; -0.0 when there is no bias, so that adding it leaves every value,
  // -0.0 included, unchanged) and the two global scales (thread 0), are
  // fetched just before the tile's first stage and stored to LDS beside it:
  // the epilogue never waits on global memory, and no register holds them
  // through the main loop.
  const bool has_bias = a.bias != nullptr;
  uint32_t bnext = 0;
  float agn = 0.0f, wgn = 0.0f;
  auto side_load = [&]() {
    const int64_t n = n0 + threadIdx.x;
    bnext = (has_bias && threadIdx.x < BN && n < a.N) ? (uint32_t)a.bias[n] : 0x8000u;
    if (threadIdx.x == 0) {
      agn = a.Ag[0];
      wgn = a.Wg[0];
    }
  };

  int t = blockIdx.x;
  setup(t);
  side_load();
  fill_load<BM, KTAIL>(fa, opa, a.K, 0);
  fill_load<BN, KTAIL>(fw, opw, a.K, 0);
  for (;;) {
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

  // prologue: stage 0 (already in registers) into LDS buffer 0, stage 1 in
  // flight in registers
  fill_store<BM>(fa, smem + T::A_CODE, smem + T::A_SCALE);
  fill_store<BN>(fw, smem + T::W_CODE, smem + T::W_SCALE);
  if (threadIdx.x < BN) reinterpret_cast<uint16_t *>(smem + T::BIAS)[threadIdx.x] = (uint16_t)bnext;
  if (threadIdx.x == 0) {
#pragma clang fp contract(off)
    *reinterpret_cast<float *>(smem + T::GG) = agn * wgn;
  }
  fill_load<BM, KTAIL>(fa, opa, a.K, 1);
  fill_load<BN, KTAIL>(fw, opw, a.K, 1);
  __syncthreads();

  frag_read<WM, WN>(fr, smem, wm, wn, r, h);
  decode_step<0, NQ>(fr, h, f0);

  for (int ks = 0; ks < nk; ++ks) {
    uint8_t *nxt = smem + ((ks + 1) & 1) * T::STAGE;
    // stage ks+1 (in registers) → LDS; fetch stage ks+2.  The buffer being
    // overwritten was last read at the start of stage ks-1, before the
    // barrier that ended it.
    fill_store<BM>(fa, nxt + T::A_CODE, nxt + T::A_SCALE);
    fill_store<BN>(fw, nxt + T::W_CODE, nxt + T::W_SCALE);
    fill_load<BM, KTAIL>(fa, opa, a.K, ks + 2);
    fill_load<BN, KTAIL>(fw, opw, a.K, ks + 2);

    decode_step<1, NQ>(fr, h, f1); mfma_step<WM, WN>(acc, f0); interleave_hint<WM, WN, 0>();
    decode_step<2, NQ>(fr, h, f0); mfma_step<WM, WN>(acc, f1); interleave_hint<WM, WN, 1>();
    decode_step<3, NQ>(fr, h, f1); mfma_step<WM, WN>(acc, f0); interleave_hint<WM, WN, 2>();
    decode_step<4, NQ>(fr, h, f0); mfma_step<WM, WN>(acc, f1); interleave_hint<WM, WN, 3>();
    decode_step<5, NQ>(fr, h, f1); mfma_step<WM, WN>(acc, f0); interleave_hint<WM, WN, 4>();
    decode_step<6, NQ>(fr, h, f0); mfma_step<WM, WN>(acc, f1); interleave_hint<WM, WN, 5>();
    decode_step<7, NQ>(fr, h, f1); mfma_step<WM, WN>(acc, f0); interleave_hint<WM, WN, 6>();
    // every wave has stored stage ks+1 and finished reading stage ks
    __syncthreads();
    frag_read<WM, WN>(fr, nxt, wm, wn, r, h);
    decode_step<0, NQ>(fr, h, f0); mfma_step<WM, WN>(acc, f1); interleave_hint<WM, WN, 7>();
  }

  // the next tile's first stage is fetched now, so its latency hides behind
  // this tile's epilogue
  const int64_t cm0 = m0, cn0 = n0;
  const int t_next = PERSIST ? t + (int)gridDim.x : ntiles;
  if (PERSIST && t_next < ntiles) {
    setup(t_next);
    side_load();
    fill_load<BM, KTAIL>(fa, opa, a.K, 0);
    fill_load<BN, KTAIL>(fw, opw, a.K, 0);
  }

  // ---- epilogue: acc[j][i][v] is C[m][n] with m = (row block i) + r,
  //      n = (column block j) + 8·(v/4) + 4·h + v%4.  Each operation rounds on
  //      its own (no fused multiply-add), as the interface states.  Stores are
  //      16 contiguous bytes per lane along the rows of C.
  uint32_t tmax = 0;                     // largest stored |bf16| pattern (tile_amax)
  {
#pragma clang fp contract(off)
    const int64_t mw = cm0 + wm * 32 * WM, nw = cn0 + wn * 32 * WN;
    const bool full = (cm0 + BM <= a.M) && (cn0 + BN <= a.N) && ((a.N & 7) == 0);
    const float gg = *reinterpret_cast<const float *>(smem + T::GG);

    float bv[WN][4][4];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * 32 * WN + 32 * j + 8 * q + 4 * h;
        const u32x2 p = *reinterpret_cast<const u32x2 *>(smem + T::BIAS + 2 * col);
        bv[j][q][0] = bf16_bits_to_f32(p.x & 0xFFFFu);
        bv[j][q][1] = bf16_bits_to_f32(p.x >> 16);
        bv[j][q][2] = bf16_bits_to_f32(p.y & 0xFFFFu);
        bv[j][q][3] = bf16_bits_to_f32(p.y >> 16);
      }

    const bool track = a.tile_amax != nullptr;
    // For column block j and q pair p, lane (r, h) holds columns 8q + 4h .. +3
    // of row r for q = 2p (X) and 2p + 1 (Y).  Swapping the upper half-wave of
    // X with the lower half-wave of Y leaves lane (r, 0) with columns
    // 16p .. +7 and lane (r, 1) with 16p + 8 .. +15: 16 contiguous bytes.
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int64_t m = mw + 32 * i + r;
      uint16_t *crow = a.C + m * a.N;
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t xy[2][2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int q = 2 * p + e;
            float o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              float y = acc[j][i][4 * q + k] * gg;
              y = y + bv[j][q][k];
              if constexpr (GELU) y = gelu_tanh(y);
              o[k] = y;
            }
            xy[e][0] = pack_bf16x2(o[0], o[1]);
            xy[e][1] = pack_bf16x2(o[2], o[3]);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(xy[0][0], xy[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(xy[0][1], xy[1][1], false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          const int64_t n = nw + 32 * j + 16 * p + 8 * h;
          if (full) {
            if (track) {
              uint32_t mx = absmax_bf16x2(absmax_bf16x2(0u, v.x), v.y);
              mx = absmax_bf16x2(absmax_bf16x2(mx, v.z), v.w);
              mx = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
              tmax = tmax > mx ? tmax : mx;
            }
            *reinterpret_cast<u32x4 *>(crow + n) = v;
          } else if (m < a.M) {
            // a tile at the edge: columns past N are neither stored nor counted
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            if (track) {
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t mag = (w[e >> 1] >> (16 * (e & 1))) & 0x7FFFu;
                if (n + e < a.N && mag > tmax) tmax = mag;
              }
            }
            if ((a.N & 7) == 0 && n + 8 <= a.N) {
              *reinterpret_cast<u32x4 *>(crow + n) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e < a.N) crow[n + e] = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
            }
          }
        }
    }
  }
  if (a.tile_amax != nullptr) {
    __shared__ uint32_t tred[kGemmThreads / 64];
    const uint32_t wmax = wave_max_u32(tmax);
    if (lane == 0) tred[wave] = wmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t mx = tred[0];
#pragma unroll
      for (int w = 1; w < kGemmThreads / 64; ++w) mx = mx > tred[w] ? mx : tred[w];
      // column-major over tiles: the tiles of one column range are contiguous
      a.tile_amax[(cn0 / BN) * tiles_m + cm0 / BM] = mx;
    }
  }
  if (t_next >= ntiles) break;
  t = t_next;
  __syncthreads();                       // every wave is done with the stage buffers and the
                                         // epilogue's LDS inputs before the next tile's fills
  }
}

// Launch of one tile shape: persistent (one workgroup per CU, the LDS ring
// and the registers allow no more, each looping over tiles w, w + grid, ...)
// except the 256x256 tile.
template <int WM, int WN>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream, int cus) {
  constexpr int BM = 64 * WM, BN = 64 * WN;
  constexpr bool P = !(WM == 4 && WN == 4);
  const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
  const int ntiles = tm * tn;
  const dim3 grid((P && ntiles > cus) ? cus : ntiles), block(kGemmThreads);
  const bool tail = a.K % kBK != 0, gelu = (a.flags & NVFP4_EPI_GELU_TANH) != 0;
  if (!tail && !gelu)
    hipLaunchKernelGGL((k_gemm<WM, WN, false, P, false>), grid, block, 0, stream, a, tm, tn);
  else if (!tail)
    hipLaunchKernelGGL((k_gemm<WM, WN, false, P, true>), grid, block, 0, stream, a, tm, tn);
  else if (!gelu)
    hipLaunchKernelGGL((k_gemm<WM, WN, true, P, false>), grid, block, 0, stream, a, tm, tn);
  else
    hipLaunchKernelGGL((k_gemm<WM, WN, true, P, true>), grid, block, 0, stream, a, tm, tn);
  return hipGetLastError();
}

// One function per tile shape, each defined in gemm_tile_<WM>x<WN>.hip.
hipError_t launch_gemm_4x4(const GemmArgs &a, hipStream_t stream, int cus);
hipError_t launch_gemm_4x3(const GemmArgs &a, hipStream_t stream, int cus);
hipError_t launch_gemm_3x4(const GemmArgs &a, hipStream_t stream, int cus);
hipError_t launch_gemm_4x2(const GemmArgs &a, hipStream_t stream, int cus);
hipError_t launch_gemm_2x4(const GemmArgs &a, hipStream_t stream, int cus);
hipError_t launch_gemm_2x2(const GemmArgs &a, hipStream_t stream, int cus);

}  // namespace nvfp4
