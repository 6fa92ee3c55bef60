// Attention over the NVFP4 KV cache, fused with its dequantisation (gfx950),
// and a bf16-K/V twin of the same kernel as the baseline.
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / 推理底座 (the KV
// cache is stored in NVFP4 and read back through a dequant kernel inside
// inference, overhead within 2 %) and 二、方法 / 多镜头注意力锚点 (a chunk attends
// to the global-sink frames, the shot-sink frames and a recent window:
// disjoint token ranges of the cache).  O = softmax(Q·Kᵀ·scale)·V per head.
//
// Work split: a workgroup owns 128 queries (4 waves x 32) of one head and one
// split of the keys; it walks its keys in tiles of 64.  Each tile is decoded
// once by the whole workgroup into LDS:
//   K as fp16 [key][d] (E2M1 · E4M3 is exact in fp16: the GEMM's convert-and-
//     scale decode), rows padded to 272 B so the fragment reads of 8 lanes
//     hit distinct banks;
//   V transposed, bf16 [d][key] (E2M1 · E4M3 exact in bf16 as well), rows
//     padded to 136 B;
//   the per-key factors g_K · scale · log2(e) and g_V of each key's append.
// Scores are computed transposed, Sᵀ = K·Qᵀ (v_mfma_f32_32x32x16_f16, Q
// converted from bf16 to fp16 once), so a lane holds 32 of one query's 64
// scores and the other 32 sit in the lane 32 apart: the row maximum is an
// in-lane reduction plus one exchange.  Online softmax in base 2 (exp2)
// against a reference that moves only when a score would exceed it by more
// than 2^kLazy (so the O rescale is rare), P times g_V rounded to bf16 (bf16
// keeps the exponent range of small probabilities), then Oᵀ += Vᵀ·Pᵀ
// (v_mfma_f32_32x32x16_bf16): the
// accumulator registers of Sᵀ are already laid out as the B operand of that
// product for the key order k = 16s + 8(i/4) + 4h + i%4, which the Vᵀ
// fragment reads follow.  The tile after the current one is fetched from
// global memory into registers (32-bit offsets, buffer loads that return 0
// past the keys) while the current one is computed; the decoded tiles
// alternate between two LDS buffers, one barrier per tile.
// With more than one split, each split writes its unnormalised O with its
// running maximum and sum, and k_attn_combine merges them.
//
// The twin (BF16) copies bf16 K and V into the same LDS layout (K kept as
// bf16, Sᵀ on the bf16 MFMA); everything else is the same code.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace nvfp4 {

constexpr int kAD = 128;                  // head_dim
constexpr int kAQ = 128;                  // queries per workgroup
constexpr int kAK = 64;                   // keys per tile
constexpr int kAThreads = 256;
constexpr int kKRow = kAD * 2 + 16;       // LDS bytes per K row (272)
constexpr int kVRow = kAK * 2 + 8;        // LDS bytes per Vᵀ row (136)
constexpr int kAttnLdsStarts = 2048;      // chunk starts kept in LDS (as int32)
constexpr float kLazy = 8.0f;             // log2 headroom of the softmax reference

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// One decoded key tile.  The workgroup keeps two: it decodes tile i+1 into
// one while its waves read tile i from the other, so one barrier per tile
// orders both.  A K-smoothed cache adds per-key append indices and the
// centre row of the tile's last append.
template <bool SMOOTH>
struct alignas(16) AttnTile {     // 16-byte multiple: both buffers keep 16-byte rows aligned
  uint8_t k[kAK * kKRow];
  uint8_t v[kAD * kVRow];
  float gk[kAK], gv[kAK];     // per key: g_K·scale·log2(e) and g_V (0 past the keys)
};
template <>
struct alignas(16) AttnTile<true> {
  uint8_t k[kAK * kKRow];
  uint8_t v[kAD * kVRow];
  float gk[kAK], gv[kAK];
  int32_t ck[kAK];              // per key the append index (−1 past the keys)
};
static_assert(sizeof(AttnTile<false>) % 16 == 0 && sizeof(AttnTile<true>) % 16 == 0,
              "tile buffers must stay 16-byte aligned");
// Chunk starts kept in LDS (as int32): fewer with K-smoothing, whose larger
// tiles and q·μ slots must leave two workgroups per CU.
template <bool SMOOTH>
constexpr int attn_lds_starts() { return SMOOTH ? 1984 : kAttnLdsStarts; }
template <bool SMOOTH>
struct AttnLds {
  AttnTile<SMOOTH> buf[2];
  int32_t starts[attn_lds_starts<SMOOTH>()];
  float bq[SMOOTH ? 2 : 1][SMOOTH ? kAThreads : 1];   // K-smoothing: two q·μ slots per thread
};
static_assert(2 * sizeof(AttnLds<true>) <= 160 * 1024 && 2 * sizeof(AttnLds<false>) <= 160 * 1024,
              "two workgroups per CU");

// The append that the previous key of this thread's slot belonged to, with
// its factors: consecutive tiles move each slot's token forward by 64, so the
// append only has to be searched again when a token leaves [lo, hi).
struct ChunkCache {
  int32_t lo = 0, hi = 0;
  float gk = 0.0f, gv = 0.0f;
  int32_t ci = -1;              // K-smoothing only
};

// Token of virtual key j (the concatenated ranges), or -1 past the keys.
__device__ __forceinline__ int64_t key_token(const AttnArgs &a, int64_t j) {
  int64_t tok = -1;
#pragma unroll
  for (int r = 0; r < kAttnMaxRanges; ++r) {
    if (r < a.n_ranges && tok < 0) {
      if (j < a.range_len[r]) tok = a.range_lo[r] + j;
      j -= a.range_len[r];
    }
  }
  return tok;
}

// Append (chunk) index of token `tok`: starts[c] <= tok < starts[c + 1].
template <typename P>
__device__ __forceinline__ int64_t attn_chunk_of(P starts, int64_t n_chunks, int64_t tok) {
  int64_t lo = 0, hi = n_chunks - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)starts[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One tile's global data in flight, per thread.
//   K part: key kk = t % 64, quarter c = t / 64 (elements 32c .. 32c+31);
//   V part: key pair kp = t % 32 (keys 2kp, 2kp+1), d-block db = t / 32
//   (elements 16db .. 16db+15); meta: threads t < 64, the token of key t.
template <bool BF16>
struct TileIn;
template <>
struct TileIn<false> {
  u32x4 kcode;
  uint32_t kscale;          // two scale bytes
  u32x2 vcode[2];
  uint32_t vscale[2];
  int32_t tok;
};
template <>
struct TileIn<true> {
  u32x4 kraw[4];            // 32 bf16
  u32x4 vraw[2][2];         // 16 bf16 per key
  int32_t tok;
};

// Token of the tile's first key when all its keys jt .. min(jt + 64, j1) − 1
// lie in one range (the usual case), else −1.  Depends only on kernel
// arguments and the tile: uniform, so it runs on the scalar unit.
__device__ __forceinline__ int64_t tile_run_token(const AttnArgs &a, int64_t jt, int64_t j1) {
  const int64_t n = (jt + kAK < j1 ? jt + kAK : j1) - jt;
  int64_t j = jt, base = -1;
  bool found = false;
#pragma unroll
  for (int r = 0; r < kAttnMaxRanges; ++r) {
    if (r < a.n_ranges && !found) {
      if (j < a.range_len[r]) {
        found = true;
        base = (j + n <= a.range_len[r]) ? a.range_lo[r] + j : -1;
      }
      j -= a.range_len[r];
    }
  }
  return base;
}

// Token of the tile's key k (−1 past the keys).
__device__ __forceinline__ int32_t tile_key_token(const AttnArgs &a, int64_t base, int64_t jt, int64_t j1, int k) {
  const int64_t j = jt + k;
  if (base >= 0) return j < j1 ? (int32_t)(base + k) : -1;
  return j < j1 ? (int32_t)key_token(a, j) : -1;
}

// Byte offset inside a buffer, or one past every buffer (the load returns 0)
// for a key past the keys.
__device__ __forceinline__ uint32_t key_offset(int32_t tok, uint32_t row_bytes, uint32_t col) {
  return tok < 0 ? 0x80000000u : __umul24((uint32_t)tok, row_bytes) + col;
}

// Tokens are below 2^24 and every tensor below 2^31 bytes (checked on the
// host), so offsets are 32-bit and the loads are buffer loads whose range
// check turns the keys past the end into zeros.
template <bool BF16>
__device__ __forceinline__ void tile_fetch(TileIn<BF16> &f, const AttnArgs &a, int h, int64_t jt,
                                           int64_t j1) {
  const int t = threadIdx.x;
  const int kk = t & 63, c = t >> 6, kp = t & 31, db = t >> 5;
  const int64_t base = tile_run_token(a, jt, j1);
  const int32_t tk = tile_key_token(a, base, jt, j1, kk);
  const int32_t tv0 = tile_key_token(a, base, jt, j1, 2 * kp);
  const int32_t tv1 = tile_key_token(a, base, jt, j1, 2 * kp + 1);
  f.tok = tk;
  if constexpr (!BF16) {
    const uint32_t hd = (uint32_t)a.heads * kAD;                     // elements per token
    const uint32_t cb = (uint32_t)a.kv_tokens * (hd / 2), sb = (uint32_t)a.kv_tokens * (hd / 16);
    const __amdgpu_buffer_rsrc_t kc = buffer_rsrc(a.kc, cb), ks = buffer_rsrc(a.ks, sb);
    const __amdgpu_buffer_rsrc_t vc = buffer_rsrc(a.vc, cb), vs = buffer_rsrc(a.vs, sb);
    const uint32_t hc = (uint32_t)h * (kAD / 2), hs = (uint32_t)h * (kAD / 16);
    f.kcode = __builtin_amdgcn_raw_buffer_load_b128(kc, (int)key_offset(tk, hd / 2, hc + 16 * c), 0, 0);
    f.kscale = __builtin_amdgcn_raw_buffer_load_b16(ks, (int)key_offset(tk, hd / 16, hs + 2 * c), 0, 0);
    f.vcode[0] = __builtin_amdgcn_raw_buffer_load_b64(vc, (int)key_offset(tv0, hd / 2, hc + 8 * db), 0, 0);
    f.vcode[1] = __builtin_amdgcn_raw_buffer_load_b64(vc, (int)key_offset(tv1, hd / 2, hc + 8 * db), 0, 0);
    f.vscale[0] = __builtin_amdgcn_raw_buffer_load_b8(vs, (int)key_offset(tv0, hd / 16, hs + db), 0, 0);
    f.vscale[1] = __builtin_amdgcn_raw_buffer_load_b8(vs, (int)key_offset(tv1, hd / 16, hs + db), 0, 0);
  } else {
    const uint32_t rowb = (uint32_t)a.ldkv * 2, nb = (uint32_t)a.kv_tokens * rowb;
    const __amdgpu_buffer_rsrc_t kb = buffer_rsrc(a.kb, nb), vb = buffer_rsrc(a.vb, nb);
    const uint32_t hb = (uint32_t)h * (kAD * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.kraw[i] = __builtin_amdgcn_raw_buffer_load_b128(kb, (int)key_offset(tk, rowb, hb + 64 * c + 16 * i), 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f.vraw[0][i] = __builtin_amdgcn_raw_buffer_load_b128(vb, (int)key_offset(tv0, rowb, hb + 32 * db + 16 * i), 0, 0);
      f.vraw[1][i] = __builtin_amdgcn_raw_buffer_load_b128(vb, (int)key_offset(tv1, rowb, hb + 32 * db + 16 * i), 0, 0);
    }
  }
}

// fp16 E2M1 · S of 8 codes: E2M1 · 2^8 by the converter, times S · 2^-8 (the
// fp16 pattern of S·2^-8 is the E4M3 byte shifted left by 7).
__device__ __forceinline__ f16x8 attn_decode8_f16(uint32_t w, uint32_t sbyte) {
  const f16x2 s = __builtin_bit_cast(f16x2, (sbyte & 0xFFu) * 0x00800080u);
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
  const auto lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const auto hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// E2M1 · S of 8 codes in binary32 (exact).
__device__ __forceinline__ void attn_decode8_f32(uint32_t w, float s, float (&o)[8]) {
  const f32x2 e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  o[0] = e0.x * s; o[1] = e0.y * s; o[2] = e1.x * s; o[3] = e1.y * s;
  o[4] = e2.x * s; o[5] = e2.y * s; o[6] = e3.x * s; o[7] = e3.y * s;
}

// Writes one fetched tile into LDS (K rows, Vᵀ rows, per-key factors).
template <bool BF16, bool SMOOTH>
__device__ __forceinline__ void tile_store(const TileIn<BF16> &f, AttnTile<SMOOTH> &L, const AttnTile<SMOOTH> *prev,
                                           const int32_t *lds_starts, ChunkCache &cc, const AttnArgs &a,
                                           int h) {
  const int t = threadIdx.x;
  const int kk = t & 63, c = t >> 6, kp = t & 31, db = t >> 5;
  uint8_t *krow = L.k + kk * kKRow + 64 * c;
  if constexpr (!BF16) {
    const uint32_t s0 = f.kscale & 0xFFu, s1 = (f.kscale >> 8) & 0xFFu;
    *reinterpret_cast<f16x8 *>(krow + 0) = attn_decode8_f16(f.kcode.x, s0);
    *reinterpret_cast<f16x8 *>(krow + 16) = attn_decode8_f16(f.kcode.y, s0);
    *reinterpret_cast<f16x8 *>(krow + 32) = attn_decode8_f16(f.kcode.z, s1);
    *reinterpret_cast<f16x8 *>(krow + 48) = attn_decode8_f16(f.kcode.w, s1);
    float v0[16], v1[16];
    {
      const float sa = e4m3_decode(f.vscale[0]), sb = e4m3_decode(f.vscale[1]);
      float tmp[8];
      attn_decode8_f32(f.vcode[0].x, sa, tmp);
#pragma unroll
      for (int i = 0; i < 8; ++i) v0[i] = tmp[i];
      attn_decode8_f32(f.vcode[0].y, sa, tmp);
#pragma unroll
      for (int i = 0; i < 8; ++i) v0[8 + i] = tmp[i];
      attn_decode8_f32(f.vcode[1].x, sb, tmp);
#pragma unroll
      for (int i = 0; i < 8; ++i) v1[i] = tmp[i];
      attn_decode8_f32(f.vcode[1].y, sb, tmp);
#pragma unroll
      for (int i = 0; i < 8; ++i) v1[8 + i] = tmp[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<uint32_t *>(L.v + (16 * db + i) * kVRow + 4 * kp) = pack_bf16x2(v0[i], v1[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4 *>(krow + 16 * i) = f.kraw[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w0 = f.vraw[0][i >> 3][(i >> 1) & 3], w1 = f.vraw[1][i >> 3][(i >> 1) & 3];
      // (key 2kp, d) in the low half, (key 2kp+1, d) in the high half
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      *reinterpret_cast<uint32_t *>(L.v + (16 * db + i) * kVRow + 4 * kp) =
          __builtin_amdgcn_perm(w1, w0, sel);
    }
  }
  if (t < kAK) {
    float gk = 0.0f, gv = 0.0f;
    int32_t kci = -1;                      // K-smoothing: the key's append (−1 past the keys)
    if (f.tok >= 0) {
      if constexpr (SMOOTH) {
        if (f.tok < cc.lo || f.tok >= cc.hi) {
          const int64_t ci = lds_starts != nullptr ? attn_chunk_of(lds_starts, a.n_chunks, (int64_t)f.tok)
                                                   : attn_chunk_of(a.chunk_start, a.n_chunks, (int64_t)f.tok);
          cc.lo = lds_starts != nullptr ? lds_starts[ci] : (int32_t)a.chunk_start[ci];
          cc.hi = lds_starts != nullptr ? lds_starts[ci + 1] : (int32_t)a.chunk_start[ci + 1];
          cc.gk = a.gscale[2 * ci] * a.qk_scale;
          cc.gv = a.gscale[2 * ci + 1];
          cc.ci = (int32_t)ci;
        }
        gk = cc.gk;
        gv = cc.gv;
        kci = cc.ci;
      } else if constexpr (!BF16) {
        if (f.tok < cc.lo || f.tok >= cc.hi) {
          const int64_t ci = lds_starts != nullptr ? attn_chunk_of(lds_starts, a.n_chunks, (int64_t)f.tok)
                                                   : attn_chunk_of(a.chunk_start, a.n_chunks, (int64_t)f.tok);
          cc.lo = lds_starts != nullptr ? lds_starts[ci] : (int32_t)a.chunk_start[ci];
          cc.hi = lds_starts != nullptr ? lds_starts[ci + 1] : (int32_t)a.chunk_start[ci + 1];
          cc.gk = a.gscale[2 * ci] * a.qk_scale;
          cc.gv = a.gscale[2 * ci + 1];
        }
        gk = cc.gk;
        gv = cc.gv;
      } else {
        gk = a.qk_scale;
        gv = 1.0f;
      }
    }
    L.gk[t] = gk;
    L.gv[t] = gv;
    if constexpr (SMOOTH) L.ck[t] = kci;
  }
}

// K-smoothing: q·μ of this lane's query (row q of Q) and the centre row of
// append c, in units of the scaled scores (times scale·log2(e)).  Each
// half-wave covers half of the dimensions (d = 16·st + 8·hh .. +7), from the
// bf16 query in memory (bf16 products are exact in the fp32 dot); one
// exchange adds the halves.  One 16-byte segment of each row in registers at
// a time: this runs while the tile loop holds its full register set.
__device__ __forceinline__ float attn_center_dot(const AttnArgs &a, int64_t q, int h, int hh, int32_t c) {
  const uint16_t *mr = a.kcenter + ((int64_t)c * a.heads + h) * kAD + 8 * hh;
  const uint16_t *qr = a.q + q * a.ldq + (int64_t)h * kAD + 8 * hh;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // 8 bytes of each row at a time; the pairs taken with shuffles of the
    // 4-element vectors (a bit cast of each 32-bit element to a bf16 pair
    // was compiled to read element 0 every time)
    const int off = 16 * (i >> 1) + 4 * (i & 1);
    const bf16x4 mv = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(mr + off));
    const bf16x4 qv = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(qr + off));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 0, 1), __builtin_shufflevector(mv, mv, 0, 1),
                                           acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(qv, qv, 2, 3), __builtin_shufflevector(mv, mv, 2, 3),
                                           acc, false);
    __builtin_amdgcn_sched_barrier(0);
  }
  acc += __shfl_xor(acc, 32, 64);
  return acc * a.qk_scale;
}

// The same q·μ from the query's fp16 fragments, the centre row read from
// memory with all its loads in flight at once (fp16 holds the bf16 centre
// exactly for |μ| in [2^-14, 65504]; smaller centres lose low bits, a change
// far below the scores' rounding).  Used where the score registers are free.
__device__ __forceinline__ float attn_center_dot_q(const AttnArgs &a, const f16x8 (&qf)[8], int h, int hh,
                                                   int32_t c) {
  const uint16_t *mr = a.kcenter + ((int64_t)c * a.heads + h) * kAD + 8 * hh;
  u32x4 raw[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) raw[st] = *reinterpret_cast<const u32x4 *>(mr + 16 * st);
  float acc = 0.0f;
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    f16x8 m;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] = (_Float16)bf16_bits_to_f32(raw[st][e] & 0xFFFFu);
      m[2 * e + 1] = (_Float16)bf16_bits_to_f32(raw[st][e] >> 16);
    }
    const f16x8 q = qf[st];
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(q, q, 0, 1), __builtin_shufflevector(m, m, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(q, q, 2, 3), __builtin_shufflevector(m, m, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(q, q, 4, 5), __builtin_shufflevector(m, m, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(q, q, 6, 7), __builtin_shufflevector(m, m, 6, 7), acc, false);
  }
  acc += __shfl_xor(acc, 32, 64);
  return acc * a.qk_scale;
}

template <bool BF16, bool SMOOTH>
__global__ void __launch_bounds__(kAThreads, 2) k_attention(AttnArgs a) {
  static_assert(!(BF16 && SMOOTH), "K-smoothing applies to the NVFP4 cache only");
  __shared__ __attribute__((aligned(16))) AttnLds<SMOOTH> L;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 31, hh = lane >> 5;
  // Work item (query block, head, split) of this workgroup, query block
  // fastest: the workgroups of one (head, split) read the same key tiles, so
  // consecutive items go to one XCD (workgroup i of a 1-D grid runs on XCD
  // i mod 8) when the grid splits evenly over the 8 XCDs, and their tiles
  // are fetched into that XCD's L2 once.
  const int64_t nwg = gridDim.x, wid = blockIdx.x;
  const int64_t item = (nwg % 8 == 0) ? (wid % 8) * (nwg / 8) + wid / 8 : wid;
  const int64_t nqb = (a.Tq + kAQ - 1) / kAQ;
  const int qb = (int)(item % nqb);
  const int h = (int)((item / nqb) % a.heads), split = (int)(item / (nqb * a.heads));
  const int64_t q = (int64_t)qb * kAQ + 32 * w + r;               // this lane's query
  const int64_t qc = q < a.Tq ? q : a.Tq - 1;
  const int64_t j0 = (int64_t)split * a.keys_per_split;
  const int64_t j1 = (j0 + a.keys_per_split < a.Tk) ? j0 + a.keys_per_split : a.Tk;

  bool starts_in_lds = false;
  if constexpr (!BF16) {
    starts_in_lds = a.n_chunks < attn_lds_starts<SMOOTH>();
    if (starts_in_lds)
      for (int64_t i = threadIdx.x; i <= a.n_chunks; i += kAThreads) L.starts[i] = (int32_t)a.chunk_start[i];
  }

  // query fragments: lane (r, hh) holds d = 16·step + 8·hh .. +7 of query q
  typedef typename std::conditional<BF16, bf16x8, f16x8>::type QFrag;
  QFrag qf[8];
  {
    const u32x4 *qp = reinterpret_cast<const u32x4 *>(a.q + qc * a.ldq + (int64_t)h * kAD + 8 * hh);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 raw = qp[2 * s];
      if constexpr (BF16) {
        qf[s] = __builtin_bit_cast(bf16x8, raw);
      } else {
        f16x8 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = raw[e];
          x[2 * e] = (_Float16)bf16_bits_to_f32(wv & 0xFFFFu);
          x[2 * e + 1] = (_Float16)bf16_bits_to_f32(wv >> 16);
        }
        qf[s] = x;
      }
    }
  }

  float m = -__builtin_huge_valf(), l = 0.0f;
  // K-smoothing: q·μ of the previous tile's last append (cbp) is in slot
  // L.bq[sp]; a tile ending in another append writes that one's into the other
  // slot, which becomes the current one after the tile
  int32_t cbp = -1;
  int sp = 0;
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.0f;

  TileIn<BF16> fin;
  ChunkCache cc;
  const int32_t *lds_starts = starts_in_lds ? L.starts : nullptr;
  tile_fetch<BF16>(fin, a, h, j0, j1);
  if constexpr (!BF16) {
    if (starts_in_lds) __syncthreads();
  }
  tile_store<BF16, SMOOTH>(fin, L.buf[0], nullptr, lds_starts, cc, a, h);
  __syncthreads();
  if (j0 + kAK < j1) tile_fetch<BF16>(fin, a, h, j0 + kAK, j1);
  int cur = 0;
  for (int64_t jt = j0; jt < j1; jt += kAK, cur ^= 1) {
    // K-smoothing: this tile's append indices, one key per lane, read before
    // the next tile's decode hides the read's latency
    int32_t ckl = -1;
    if constexpr (SMOOTH) ckl = L.buf[cur].ck[lane];
    // decode the next tile into the other buffer (its loads were issued one
    // tile ago), then fetch the one after it
    if (jt + kAK < j1) {
      tile_store<BF16, SMOOTH>(fin, L.buf[cur ^ 1], &L.buf[cur], lds_starts, cc, a, h);
      if (jt + 2 * kAK < j1) tile_fetch<BF16>(fin, a, h, jt + 2 * kAK, j1);
    }
    const AttnTile<SMOOTH> &B = L.buf[cur];

    // Keys of a smoothed cache are E2M1·S·g + μ: each score gains q·μ of its
    // key's append.  Every wave reads the tile's append indices (one key per
    // lane) and finds whether one append holds the tile and which append its
    // last key is in; q·μ of that last append is computed here, before the
    // score registers are in use, unless the previous tile ended in the same
    // append, and a tile that starts in the previous tile's append finds that
    // value in the other slot.  Any other append (a tile over three or more,
    // or the first tile of a split that starts in another append) is read
    // from memory where it is needed.
    int32_t cl = -1, scl = 0;
    bool one_append = false;
    if constexpr (SMOOTH) {
      const uint64_t valid = __ballot(ckl >= 0);                  // a prefix of the keys
      const int32_t ck0 = __builtin_amdgcn_readfirstlane(ckl);
      cl = __builtin_amdgcn_readlane(ckl, 63 - __builtin_clzll(valid));
      one_append = __ballot(ckl >= 0 && ckl != ck0) == 0;
      scl = cl != cbp ? 1 - sp : sp;
      if (cl != cbp) L.bq[scl][threadIdx.x] = attn_center_dot_q(a, qf, h, hh, cl);
    }
    // Sᵀ = K·Qᵀ: lane (query r, hh) gets keys 32kb + 8(v/4) + 4hh + v%4
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t *kr = B.k + (32 * kb + r) * kKRow + 16 * hh;
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(kr + 32 * st);
        if constexpr (BF16)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, raw), qf[st], acc, 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, raw), qf[st], acc, 0, 0, 0);
      }
      s[kb] = acc;
    }
    // Softmax in base 2 against a reference m that moves lazily: m (and with
    // it O and l) moves only when some query of the wave sees a scaled score
    // more than 2^kLazy above it, so p = 2^(s·g_K − m) stays below 2^kLazy.
    // Any reference gives the same result: O and l carry the same factor, and
    // the split merge uses m.  The exponent t = s·g_K − m is formed by one FMA
    // (before the first reference, t = s·g_K); the tile's largest t decides
    // whether m moves, and a move shifts t by the same amount.  Keys past the
    // split (only in its last tile) score −inf.
    const int kvalid = (j1 - jt) < kAK ? (int)(j1 - jt) : kAK;
    const bool no_ref = m == -__builtin_huge_valf();
    const float off = no_ref ? 0.0f : -m;
    float mt = -__builtin_huge_valf();
    if constexpr (SMOOTH) {
      if (one_append) {
        // one append holds the tile: the term q·μ of the scaled score
        const float bq = L.bq[scl][threadIdx.x] + off;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int key0 = 32 * kb + 8 * g4 + 4 * hh;
            const f32x4 gk4 = *reinterpret_cast<const f32x4 *>(&B.gk[key0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float tv = key0 + e < kvalid ? __builtin_fmaf(s[kb][4 * g4 + e], gk4[e], bq)
                                                 : -__builtin_huge_valf();
              s[kb][4 * g4 + e] = tv;
              mt = __builtin_fmaxf(mt, tv);
            }
          }
      } else {
        uint64_t runs = __ballot(lane == 0 || ckl != B.ck[lane == 0 ? 0 : lane - 1]);
        while (runs != 0) {
          const int k0 = __builtin_ctzll(runs);
          runs &= runs - 1;
          const int k1 = runs != 0 ? __builtin_ctzll(runs) : kAK;
          const int32_t c = __builtin_amdgcn_readfirstlane(B.ck[k0]);
          if (c < 0) continue;                       // keys past the end (masked below)
          const float b = c == cl ? L.bq[scl][threadIdx.x]
                                  : (c == cbp ? L.bq[sp][threadIdx.x] : attn_center_dot(a, qc, h, hh, c));
          const float bi = b / B.gk[k0];             // enters before the key factor
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = 32 * kb + 8 * g4 + 4 * hh + e;
                if (key >= k0 && key < k1) s[kb][4 * g4 + e] += bi;
              }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int key0 = 32 * kb + 8 * g4 + 4 * hh;
            const f32x4 gk4 = *reinterpret_cast<const f32x4 *>(&B.gk[key0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float tv = key0 + e < kvalid ? __builtin_fmaf(s[kb][4 * g4 + e], gk4[e], off)
                                                 : -__builtin_huge_valf();
              s[kb][4 * g4 + e] = tv;
              mt = __builtin_fmaxf(mt, tv);
            }
          }
      }
    } else if (kvalid == kAK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 gk4 = *reinterpret_cast<const f32x4 *>(&B.gk[32 * kb + 8 * g4 + 4 * hh]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float tv = __builtin_fmaf(s[kb][4 * g4 + e], gk4[e], off);
            s[kb][4 * g4 + e] = tv;
            mt = __builtin_fmaxf(mt, tv);
          }
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int key0 = 32 * kb + 8 * g4 + 4 * hh;
          const f32x4 gk4 = *reinterpret_cast<const f32x4 *>(&B.gk[key0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float tv = key0 + e < kvalid ? __builtin_fmaf(s[kb][4 * g4 + e], gk4[e], off)
                                               : -__builtin_huge_valf();
            s[kb][4 * g4 + e] = tv;
            mt = __builtin_fmaxf(mt, tv);
          }
        }
    }
    mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__builtin_amdgcn_ballot_w64(no_ref || mt > kLazy) != 0) {
      // before the first reference mt is the largest s·g_K itself (finite:
      // the first key of a split's first tile is always valid)
      const float d = no_ref ? mt : __builtin_fmaxf(mt, 0.0f);
      const float alpha = no_ref ? 1.0f : __builtin_amdgcn_exp2f(-d);
      l *= alpha;
      m = no_ref ? d : m + d;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] -= d;
    }
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = __builtin_amdgcn_exp2f(s[kb][v]);
        s[kb][v] = pv;
        psum += pv;
      }
    l += psum;
    // Pᵀ fragments (p·g_V rounded to bf16): slice sl holds keys
    // 16sl + 8(i/4) + 4hh + i%4 for i = 0..7, registers 8(sl%2) + i of s[sl/2]
    bf16x8 pf[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int kb = sl >> 1, v0 = 8 * (sl & 1);
      const f32x4 ga = *reinterpret_cast<const f32x4 *>(&B.gv[32 * kb + 8 * (v0 / 4) + 4 * hh]);
      const f32x4 gb = *reinterpret_cast<const f32x4 *>(&B.gv[32 * kb + 8 * (v0 / 4 + 1) + 4 * hh]);
      u32x4 pk;
      pk.x = pack_bf16x2(s[kb][v0 + 0] * ga[0], s[kb][v0 + 1] * ga[1]);
      pk.y = pack_bf16x2(s[kb][v0 + 2] * ga[2], s[kb][v0 + 3] * ga[3]);
      pk.z = pack_bf16x2(s[kb][v0 + 4] * gb[0], s[kb][v0 + 5] * gb[1]);
      pk.w = pack_bf16x2(s[kb][v0 + 6] * gb[2], s[kb][v0 + 7] * gb[3]);
      pf[sl] = __builtin_bit_cast(bf16x8, pk);
    }
    // Oᵀ += Vᵀ·Pᵀ: lane (d = 32db + r, hh) reads keys 16sl + 4hh .. +3 and 16sl + 8 + 4hh .. +3
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk) {
      const uint8_t *vr = B.v + (32 * dbk + r) * kVRow + 8 * hh;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr + 32 * sl);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 32 * sl + 16);
        const u32x4 vv = {lo.x, lo.y, hi.x, hi.y};
        o[dbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[sl], o[dbk], 0, 0, 0);
      }
    }
    if constexpr (SMOOTH) {
      cbp = cl;
      sp = scl;
    }
    // every wave has read tile `cur` and stored the next one
    __syncthreads();
  }

  // both half-waves hold the same query; their sums cover disjoint keys
  const float lt = l + __shfl_xor(l, 32, 64);
  if (q >= a.Tq) return;
  if (a.part_o == nullptr) {
    const float inv = 1.0f / lt;
    uint16_t *orow = a.o + q * a.ldo + (int64_t)h * kAD;
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dbk + 8 * g4 + 4 * hh;
        const u32x2 pk = {pack_bf16x2(o[dbk][4 * g4] * inv, o[dbk][4 * g4 + 1] * inv),
                          pack_bf16x2(o[dbk][4 * g4 + 2] * inv, o[dbk][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2 *>(orow + d) = pk;
      }
  } else {
    const int64_t row = ((int64_t)split * a.Tq + q) * a.heads + h;
    float *po = a.part_o + row * kAD;
#pragma unroll
    for (int dbk = 0; dbk < 4; ++dbk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dbk + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4 *>(po + d) =
            f32x4{o[dbk][4 * g4], o[dbk][4 * g4 + 1], o[dbk][4 * g4 + 2], o[dbk][4 * g4 + 3]};
      }
    if (hh == 0) *reinterpret_cast<f32x2 *>(a.part_ml + 2 * row) = f32x2{m, lt};
  }
}

// Merges the splits of one (query, head) row per 128 threads (one per d):
// O = Σ_s O_s · 2^(m_s − M) / Σ_s l_s · 2^(m_s − M), M = max_s m_s.
__global__ void __launch_bounds__(kAThreads) k_attn_combine(AttnArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);       // q·heads + h
  const int d = threadIdx.x & 127;
  if (row >= a.Tq * a.heads) return;
  const int64_t rows = a.Tq * a.heads;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = a.part_ml[2 * (s * rows + row)];
    M = M > ms ? M : ms;
  }
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = a.part_ml[2 * (s * rows + row)], ls = a.part_ml[2 * (s * rows + row) + 1];
    const float wgt = __builtin_amdgcn_exp2f(ms - M);
    num += a.part_o[(s * rows + row) * kAD + d] * wgt;
    den += ls * wgt;
  }
  const int64_t qi = row / a.heads, h = row - qi * a.heads;
  const float val = num / den;
  a.o[qi * a.ldo + h * kAD + d] = (uint16_t)(pack_bf16x2(val, 0.0f) & 0xFFFFu);
}

// Key splits per (query tile, head): the fewest that fill whole rounds of the
// 512 workgroup slots of an MI355X (256 CUs, two workgroups each) to at least
// 90 %, else the best filling; at least 8 key tiles per split, at most 32
// splits.  Depends only on the shapes, so the workspace size does too.
int64_t attention_splits(int64_t Tq, int64_t heads, int64_t Tk) {
  constexpr int64_t kSlots = 512;
  const int64_t tiles = ((Tq + kAQ - 1) / kAQ) * heads;
  int64_t most = Tk / (8 * kAK);
  if (most > 32) most = 32;
  if (most < 1) return 1;
  int64_t best = 1;
  double best_fill = 0.0;
  for (int64_t n = 1; n <= most; ++n) {
    const int64_t wgs = tiles * n;
    const int64_t rounds = (wgs + kSlots - 1) / kSlots;
    const double fill = (double)wgs / (double)(rounds * kSlots);
    if (fill >= 0.9) return n;
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = n;
    }
  }
  return best;
}

int64_t attention_keys_per_split(int64_t Tk, int64_t nsplit) {
  const int64_t per = (Tk + nsplit - 1) / nsplit;
  return (per + kAK - 1) / kAK * kAK;
}

hipError_t launch_attention(const AttnArgs &a, bool bf16, hipStream_t stream) {
  const int64_t items = (a.Tq + kAQ - 1) / kAQ * a.heads * a.nsplit;
  if (items > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)items);
  if (bf16)
    hipLaunchKernelGGL((k_attention<true, false>), grid, dim3(kAThreads), 0, stream, a);
  else if (a.kcenter != nullptr)
    hipLaunchKernelGGL((k_attention<false, true>), grid, dim3(kAThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((k_attention<false, false>), grid, dim3(kAThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.part_o == nullptr) return e;
  const int64_t rows = a.Tq * a.heads;
  hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((rows + 1) / 2)), dim3(kAThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
