// NVFP4 quantiser kernels (gfx950).
//
// Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成", 二、方法 / NVFP4 量化格式
// (E2M1 elements, one E4M3 scale per 16 elements, one FP32 tensor scale) and
// NVFP4 训练的工程细节 (1-D block scaling of activations).  The same kernels
// quantise the KV cache in place (二、方法 / 推理底座).
//
// Two implementations of the same arithmetic:
//
//   resident (one launch, the input is read once)
//             at most one workgroup per CU; every lane loads whole 16-element
//             blocks (32 bytes each) and keeps them in registers; each
//             workgroup publishes its |x| maximum in a 64-bit (call epoch,
//             amax) slot and then polls all slots, so every workgroup derives
//             A itself; then it encodes its registers, one 8-byte code store
//             and one scale byte per block.  Used whenever the tensors fit in
//             the registers of such a grid (plus LDS for one large tensor,
//             whose remainder is streamed, or for a K/V pair of up to ~100
//             MB); a workgroup whose wait for A expires reads the shares of
//             the workgroups it has not heard from itself, so the result does
//             not depend on residency.
//   two-pass  k_amax (grid-stride max of |x|, one partial per workgroup),
//             then k_encode (every workgroup folds the partials and encodes);
//             lanes take consecutive 16-element blocks, four per round.  Used
//             for larger tensors, and by itself (with the maxima a GEMM
//             epilogue recorded) for a linear layer's NVFP4 hand-off.
//
// The block amax is taken on the 15-bit magnitude pattern, which orders like
// the value for finite bf16.  With K % 32 == 0 a 32-element unit never crosses
// a row, and the outputs are dense in unit order; the input may be row-strided
// (a KV append can read the K and V column slices of a fused QKV output in
// place).
#include <atomic>
#include <mutex>

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
  uint64_t *slots;       // resident launch: kResidentSlots (epoch, max) slots
  uint32_t *partials;    // two-pass launch: kAmaxBlocks partial maxima
  int64_t units;         // elements / 32
  uint32_t units_per_row;
  int64_t ld;            // input elements between row starts
  const uint16_t *center;  // K-smoothing: bf16 per column, subtracted on load (or null)
};

// First 16-byte chunk of unit u in the (possibly row-strided) input.
__device__ __forceinline__ const u32x4 *unit_src(const QuantTensor &T, int64_t u) {
  const uint32_t row = (uint32_t)u / T.units_per_row;
  const uint32_t col = (uint32_t)u - row * T.units_per_row;
  return reinterpret_cast<const u32x4 *>(T.x + (int64_t)row * T.ld + 32 * (int64_t)col);
}
// First 16-byte half of 16-element block b of the tensor (unit order).
__device__ __forceinline__ const u32x4 *block_src(const QuantTensor &T, int64_t b) {
  return unit_src(T, b >> 1) + 2 * (b & 1);
}

// K-smoothing: block b's 16 elements minus the centres of their columns,
// bf16_rne(fl32(x − μ)) (a no-op without centres).
__device__ __forceinline__ void center_block(const QuantTensor &T, int64_t b, uint32_t (&w)[8]) {
  if (T.center == nullptr) return;
  const uint32_t cb = (uint32_t)b % (2u * T.units_per_row);          // block within its row
  const u32x4 *m = reinterpret_cast<const u32x4 *>(T.center + 16 * cb);
  const u32x4 m0 = m[0], m1 = m[1];
  const uint32_t mu[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w[k] = pack_bf16x2(bf16_bits_to_f32(w[k] & 0xFFFFu) - bf16_bits_to_f32(mu[k] & 0xFFFFu),
                       bf16_bits_to_f32(w[k] >> 16) - bf16_bits_to_f32(mu[k] >> 16));
}

// Block b of the tensor as 8 bf16 pairs (two 16-byte loads), centred when
// the tensor has centres (CENTER: only the kernels that take K/V pairs carry
// that code; the single-tensor ones never get centres).
template <bool CENTER = true>
__device__ __forceinline__ void load_block(const QuantTensor &T, int64_t b, uint32_t (&w)[8]) {
  const u32x4 *p = block_src(T, b);
  const u32x4 lo = p[0], hi = p[1];
  w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
  w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
  if constexpr (CENTER) center_block(T, b, w);
}

// Largest magnitude (bf16 pattern) of 8 bf16 pairs.
__device__ __forceinline__ uint32_t absmax16(const uint32_t (&w)[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = absmax_bf16x2(m, w[j]);
  return (m & 0xFFFFu) > (m >> 16) ? (m & 0xFFFFu) : (m >> 16);
}

// Two-pass kernels: each thread takes kTwoPassU 16-element blocks per round,
// consecutive lanes on consecutive blocks.
constexpr int kTwoPassU = 4;

struct QuantArgs {
  QuantTensor t[2];
  ChunkMark mark;        // chunk_start == nullptr: nothing to record
};

__global__ void __launch_bounds__(kThreads) k_amax(QuantArgs args) {
  const QuantTensor &T = args.t[blockIdx.y];
  const int64_t nb = 2 * T.units;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kTwoPassU;
  uint32_t m = 0;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kTwoPassU + threadIdx.x; base < nb; base += stride) {
    uint32_t w[kTwoPassU][8];
#pragma unroll
    for (int i = 0; i < kTwoPassU; ++i) {
      const int64_t b = base + (int64_t)i * kThreads;
      if (b < nb) {
        load_block(T, b, w[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[i][e] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < kTwoPassU; ++i) {
      const uint32_t a = absmax16(w[i]);
      m = m > a ? m : a;
    }
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
    T.partials[blockIdx.x] = r;
  }
}

// Folds the amax partials of one tensor into g.  Every block does this.
__device__ __forceinline__ float block_global_scale(const QuantTensor &T, int nparts) {
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
  return (r == 0) ? 1.0f : bf16_bits_to_f32(r) / kGlobalDivisor;   // fl(A / 2688)
}

// E2M1 codes of the bf16 pair w scaled by r, written into byte SEL of old
// (first element in the low nibble).  The converter rounds to nearest even,
// saturates at ±6 and keeps the sign of zero; its scale operand is 1.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t old, uint32_t w, float r) {
  const float x0 = bf16_bits_to_f32(w & 0xFFFFu), x1 = bf16_bits_to_f32(w >> 16);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0 * r, x1 * r, 1.0f, SEL);
}

// E2M1 codes of one 16-element block (8 bf16 pairs) scaled by r: element 2j
// in the low nibble of byte j, elements 0..7 in lo, 8..15 in hi.
__device__ __forceinline__ void encode_codes(const uint32_t (&w)[8], float r, uint32_t &lo,
                                             uint32_t &hi) {
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
}

// Encodes one 16-element block held as 8 bf16 pairs whose largest magnitude
// is bm; returns the scale byte and writes the 8 code bytes to lo/hi.
__device__ __forceinline__ uint32_t encode_block16(const uint32_t (&w)[8], uint32_t bm,
                                                   const BlockScaler &bsc, uint32_t &lo,
                                                   uint32_t &hi) {
  const uint32_t S = bsc.scale_byte(bm);
  encode_codes(w, bsc.recip(S), lo, hi);
  return S;
}

// Squared error of elements 2J, 2J+1 of an encoding, added to err in index
// order: deq = fl(fl(E2M1·S)·g) with the code's sign, e = fl(x − deq),
// err = fl(err + fl(e·e)).  Every operation rounds on its own.
template <int J>
__device__ __forceinline__ float err_pair(float err, uint32_t w, uint32_t codes, float sv, float g) {
#pragma clang fp contract(off)
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, J & 3);   // signed E2M1
  const float x0 = bf16_bits_to_f32(w & 0xFFFFu), x1 = bf16_bits_to_f32(w >> 16);
  const float e0 = x0 - (v.x * sv) * g;
  err = err + e0 * e0;
  const float e1 = x1 - (v.y * sv) * g;
  err = err + e1 * e1;
  return err;
}

__device__ __forceinline__ float block_err(const uint32_t (&w)[8], uint32_t lo, uint32_t hi,
                                           uint32_t S, float g) {
  const float sv = e4m3_decode(S);
  float err = 0.0f;
  err = err_pair<0>(err, w[0], lo, sv, g);
  err = err_pair<1>(err, w[1], lo, sv, g);
  err = err_pair<2>(err, w[2], lo, sv, g);
  err = err_pair<3>(err, w[3], lo, sv, g);
  err = err_pair<4>(err, w[4], hi, sv, g);
  err = err_pair<5>(err, w[5], hi, sv, g);
  err = err_pair<6>(err, w[6], hi, sv, g);
  err = err_pair<7>(err, w[7], hi, sv, g);
  return err;
}

// Adaptive {4, 6} selection: the block is encoded with its amax mapped to 6
// and to 4; the encoding with the smaller binary32 squared error is kept,
// ties to 6 (identical scale bytes give identical codes, so no error is
// computed for them).
__device__ __forceinline__ uint32_t encode_block16_46(const uint32_t (&w)[8], uint32_t bm,
                                                      const BlockScaler &b6, const BlockScaler &b4,
                                                      uint32_t &lo, uint32_t &hi) {
  const uint32_t S6 = b6.scale_byte(bm), S4 = b4.scale_byte(bm);
  encode_codes(w, b6.recip(S6), lo, hi);
  if (S4 == S6) return S6;
  uint32_t lo4, hi4;
  encode_codes(w, b4.recip(S4), lo4, hi4);
  const float e6 = block_err(w, lo, hi, S6, b6.g), e4 = block_err(w, lo4, hi4, S4, b4.g);
  if (e4 < e6) {
    lo = lo4;
    hi = hi4;
    return S4;
  }
  return S6;
}

// One block in the selected mode.
template <bool ADAPT>
__device__ __forceinline__ uint32_t encode_any(const uint32_t (&w)[8], uint32_t bm,
                                               const BlockScaler &b6, const BlockScaler &b4,
                                               uint32_t &lo, uint32_t &hi) {
  return ADAPT ? encode_block16_46(w, bm, b6, b4, lo, hi) : encode_block16(w, bm, b6, lo, hi);
}

template <bool ADAPT>
__global__ void __launch_bounds__(kThreads) k_encode(QuantArgs args, int nparts) {
  const QuantTensor &T = args.t[blockIdx.y];
  const float g = block_global_scale(T, nparts);
  const BlockScaler b6(g, kE2M1Max), b4(g, 4.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *T.gscale = g;
    if (blockIdx.y == 0 && args.mark.chunk_start != nullptr) {
      args.mark.chunk_start[args.mark.index] = args.mark.value;
      if (args.mark.index == 1) args.mark.chunk_start[0] = 0;
    }
  }
  const int64_t nb = 2 * T.units;
  const int64_t stride = (int64_t)gridDim.x * kThreads * kTwoPassU;
  u32x2 *codes = reinterpret_cast<u32x2 *>(T.codes);
  uint8_t *scales = reinterpret_cast<uint8_t *>(T.scales);
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kTwoPassU + threadIdx.x; base < nb; base += stride) {
    uint32_t w[kTwoPassU][8];
#pragma unroll
    for (int i = 0; i < kTwoPassU; ++i) {
      const int64_t b = base + (int64_t)i * kThreads;
      if (b < nb) {
        load_block(T, b, w[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[i][e] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < kTwoPassU; ++i) {
      const int64_t b = base + (int64_t)i * kThreads;
      uint32_t lo, hi;
      const uint32_t S = encode_any<ADAPT>(w[i], absmax16(w[i]), b6, b4, lo, hi);
      if (b < nb) {
        codes[b] = u32x2{lo, hi};
        scales[b] = (uint8_t)S;
      }
    }
  }
}

// Two-dimensional blocks: 16 rows x 16 elements along K share one scale byte,
// stored on each of the 16 rows (the [rows, K/16] scale layout is unchanged,
// so the GEMM reads such weights as it reads any).  One thread per tile,
// consecutive threads on consecutive column blocks of a row group, so every
// load of a wave covers consecutive memory.  Pass 1 takes the tile's amax;
// pass 2 reads the 16 row blocks again (from L1/L2) and encodes them with the
// tile's scale.  Source: 二、方法 / NVFP4 训练的工程细节 (weight blocks along two
// dimensions, so W and its transpose share one quantisation).
__global__ void __launch_bounds__(kThreads) k_encode_2d(QuantArgs args, int nparts, int64_t rows) {
  const QuantTensor &T = args.t[0];
  const float g = block_global_scale(T, nparts);   // has a barrier: before any return
  const BlockScaler b6(g, kE2M1Max);
  if (blockIdx.x == 0 && threadIdx.x == 0) *T.gscale = g;
  const int64_t nbc = 2 * (int64_t)T.units_per_row;                 // 16-blocks per row
  const int64_t tile = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (tile >= (rows + 15) / 16 * nbc) return;
  const int64_t grp = tile / nbc, bc = tile - grp * nbc;
  const int64_t r0 = 16 * grp, r1 = (r0 + 16 < rows) ? r0 + 16 : rows;
  uint32_t am = 0;
  for (int64_t r = r0; r < r1; ++r) {
    uint32_t w[8];
    load_block<false>(T, r * nbc + bc, w);
    const uint32_t a = absmax16(w);
    am = am > a ? am : a;
  }
  const uint32_t S = b6.scale_byte(am);
  const float rc = b6.recip(S);
  u32x2 *codes = reinterpret_cast<u32x2 *>(T.codes);
  uint8_t *scales = reinterpret_cast<uint8_t *>(T.scales);
  for (int64_t r = r0; r < r1; ++r) {
    uint32_t w[8], lo, hi;
    const int64_t b = r * nbc + bc;
    load_block<false>(T, b, w);
    encode_codes(w, rc, lo, hi);
    codes[b] = u32x2{lo, hi};
    scales[b] = (uint8_t)S;
  }
}

// ---------------------------------------------------------------------------
// Resident single-pass quantiser.

// Slot words: bits 63..16 the call's epoch, bits 15..0 a bf16 magnitude.
constexpr uint64_t kEpochMask = (uint64_t(1) << 48) - 1;
constexpr uint64_t kWaitTicks = 100000;       // 1 ms of the 100 MHz real-time counter
static std::atomic<uint64_t> g_wait_ticks{kWaitTicks};

__device__ __forceinline__ uint64_t load_slot(const uint64_t *slot) {
  return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Largest value of m over the NT threads of the workgroup (red: NT/64 words).
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t m, uint32_t *red) {
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = r > red[w] ? r : red[w];
  return r;
}

constexpr int kResThreads = 1024;            // one workgroup per CU
constexpr int kStreamU = 2;                   // streamed blocks per thread per round
constexpr int kLdsBlocks = 4;                 // LDS-resident blocks per thread (128 KB): STREAM 4, PAIRLDS 2 per tensor

// This thread's part of the |x| maximum of workgroup p's share of a tensor
// (the blocks that workgroup p loads, including its streamed chunks): read by
// a workgroup whose wait for p's slot expired.
template <bool STREAM, bool CENTER>
__device__ uint32_t share_max(const QuantTensor &T, int p, int u, int nwg) {
  const int64_t nb = 2 * T.units;
  uint32_t m = 0;
  for (int i = 0; i < u; ++i) {
    const int64_t b = ((int64_t)p * u + i) * kResThreads + threadIdx.x;
    if (b < nb) {
      uint32_t w[8];
      load_block<CENTER>(T, b, w);
      const uint32_t a = absmax16(w);
      m = m > a ? m : a;
    }
  }
  if constexpr (STREAM) {
    const int64_t cstride = (int64_t)nwg * kResThreads;
    for (int64_t b = cstride * u + (int64_t)p * kResThreads + threadIdx.x; b < nb; b += cstride) {
      uint32_t w[8];
      load_block<CENTER>(T, b, w);
      const uint32_t a = absmax16(w);
      m = m > a ? m : a;
    }
  }
  return m;
}

// Workgroup k owns, in each of the NJ tensors, the 16-element blocks
// (k·u + i)·1024 + thread, i < u <= UMAX; a thread loads a block as two
// 16-byte halves and keeps it in registers.  Each workgroup publishes its
// maximum per tensor in slot k, then polls all slots of the grid (one load per
// thread), so every workgroup derives A itself after one round trip.  The wait
// is bounded: if it expires (the grid was not resident all at once), the
// workgroup reads the shares of the workgroups whose slots it has not seen
// itself, which yields the same A, so the result never depends on scheduling.
//
// The epoch that tags the slots of a call: every call leaves all
// kResidentSlots slots of each of its tensors with one tag (workgroup k
// publishes slot k and stamps slots k + i·nwg, i >= 1, with its epoch), so
// workgroup k takes one more than the largest tag in its own slot of each
// tensor.  Only workgroup k writes slot k during a call, so every workgroup of
// a call derives the same epoch, whenever it runs, and that epoch is above
// every tag a slot of the call's tensors holds: a slot left by an earlier call
// is never taken for a current one, whatever the grid sizes of the calls and
// whichever tensors they paired.  Nothing is shared but the slots, so no
// arrival count is needed.  Because the tags live in device memory, each
// replay of a captured graph gets a new epoch.
// STREAM (one tensor, UMAX = 8, u = 8 + kLdsBlocks): the tensor is larger
// than the registers of the grid hold.  Its first nwg·1024·u blocks stay
// resident, blocks 0..7 of a thread in registers as above and blocks
// 8..8+kLdsBlocks−1 in LDS (loaded first, while the registers are free, each
// thread reading back only what it stored); the rest is dealt to the
// workgroups in chunks of 1024 consecutive blocks, read once for the maximum
// and once more to encode (from the MALL when it fits there).  Only that
// remainder is read twice, where the two-pass kernels read the whole tensor
// twice.
// PAIRLDS (a K/V pair, UMAX = 4, u <= 4 + kLdsBlocks/2): blocks 4 and 5 of each
// tensor are held in LDS the same way, so a pair of up to ~100 MB (an 8-frame
// KV chunk of 7040 tokens x 24 heads x 128, 二、方法 / 推理底座) is read once;
// K's LDS blocks are centred when they are first read back and stored back
// centred.
template <int NJ, int UMAX, bool ADAPT, bool STREAM = false, bool PAIRLDS = false>
__global__ void __launch_bounds__(kResThreads) k_quant_resident(QuantArgs args,
                                                                int u, uint64_t wait_ticks) {
  static_assert(!PAIRLDS || (NJ == 2 && !STREAM), "LDS-resident pairs are K/V pairs");
  const int k = blockIdx.x, nwg = gridDim.x;
  // the call's epoch: one more than the largest tag of this workgroup's slots
  uint64_t epoch = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint64_t e = load_slot(args.t[j].slots + k) >> 16;
    epoch = epoch > e ? epoch : e;
  }
  epoch = (epoch + 1) & kEpochMask;
  if (epoch == 0) epoch = 1;
  constexpr int NW = kResThreads / 64;
  constexpr bool LDSRES = STREAM || PAIRLDS;
  constexpr int ULDS = LDSRES ? kLdsBlocks / NJ : 0;     // LDS-resident blocks per thread per tensor
  __shared__ uint32_t red[NJ][NW], red2[NJ][NW];
  __shared__ uint64_t miss[NJ][NW];
  // LDS-resident blocks, [tensor·ULDS + block][half][thread]: each wave's
  // 16-byte stores and loads cover consecutive addresses
  __shared__ u32x4 lds_blk[LDSRES ? 2 * kLdsBlocks * kResThreads : 1];

  // LDS-resident blocks: loaded straight into LDS (no registers held), lane
  // l of a wave into slot l of the wave's 64-slot run; lanes past the tensor
  // load nothing, and their slots are never read
  if constexpr (LDSRES) {
    [[maybe_unused]] const int wave_base = threadIdx.x & ~63;          // device pass only
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const QuantTensor &T = args.t[j];
#pragma unroll
      for (int i = 0; i < ULDS; ++i) {
        const int64_t b = ((int64_t)k * u + UMAX + i) * kResThreads + threadIdx.x;
        [[maybe_unused]] const int slot = j * ULDS + i;
        if (UMAX + i < u && b < 2 * T.units) {
          [[maybe_unused]] const u32x4 *p = block_src(T, b);
#if defined(__HIP_DEVICE_COMPILE__)      // device-only builtin; the host pass only parses the kernel
          __builtin_amdgcn_global_load_lds(p, &lds_blk[(2 * slot) * kResThreads + wave_base], 16, 0, 0);
          __builtin_amdgcn_global_load_lds(p + 1, &lds_blk[(2 * slot + 1) * kResThreads + wave_base], 16, 0,
                                           0);
#endif
        }
      }
    }
  }

  // (block maxima are recomputed at encode time rather than kept: eight
  // registers fewer through the poll)
  uint32_t w[NJ][UMAX][8];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const QuantTensor &T = args.t[j];
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const int64_t b = ((int64_t)k * u + i) * kResThreads + threadIdx.x;
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (i < u && b < 2 * T.units) {
        const u32x4 *p = block_src(T, b);
        lo = p[0];
        hi = p[1];
      }
      w[j][i][0] = lo.x; w[j][i][1] = lo.y; w[j][i][2] = lo.z; w[j][i][3] = lo.w;
      w[j][i][4] = hi.x; w[j][i][5] = hi.y; w[j][i][6] = hi.z; w[j][i][7] = hi.w;
    }
  }
  // K-smoothing (K/V pairs only): centre the blocks once all loads are in
  // flight (blocks past the tensor stay 0: never encoded, maximum unused)
  if constexpr (NJ == 2) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < UMAX; ++i) {
        const int64_t b = ((int64_t)k * u + i) * kResThreads + threadIdx.x;
        if (args.t[j].center != nullptr && i < u && b < 2 * args.t[j].units) center_block(args.t[j], b, w[j][i]);
      }
  }
  // streamed blocks (STREAM): b = nwg·u·1024 + (s·nwg + k)·1024 + thread
  uint32_t ms = 0, ml[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) ml[j] = 0;
  if constexpr (STREAM) {
    const QuantTensor &T = args.t[0];
    const int64_t nb = 2 * T.units, cstride = (int64_t)nwg * kResThreads;
    const int64_t chunk0 = cstride * u + (int64_t)k * kResThreads + threadIdx.x;
    for (int64_t b0 = chunk0; b0 < nb; b0 += kStreamU * cstride) {
      uint32_t v[kStreamU][8];
#pragma unroll
      for (int i = 0; i < kStreamU; ++i) {
        const int64_t b = b0 + i * cstride;
        if (b < nb) {
          load_block<false>(T, b, v[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[i][e] = 0u;
        }
      }
#pragma unroll
      for (int i = 0; i < kStreamU; ++i) {
        const uint32_t am = absmax16(v[i]);
        ms = ms > am ? ms : am;
      }
    }
  }
  if constexpr (LDSRES) {
    // every load of this wave has landed (the direct-to-LDS ones included)
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_s_waitcnt(0);
#endif
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const QuantTensor &T = args.t[j];
#pragma unroll
      for (int i = 0; i < ULDS; ++i) {
        const int64_t b = ((int64_t)k * u + UMAX + i) * kResThreads + threadIdx.x;
        const int slot = j * ULDS + i;
        if (UMAX + i < u && b < 2 * T.units) {
          u32x4 lo4 = lds_blk[(2 * slot) * kResThreads + threadIdx.x];
          u32x4 hi4 = lds_blk[(2 * slot + 1) * kResThreads + threadIdx.x];
          uint32_t wv[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
          if constexpr (PAIRLDS) {
            if (T.center != nullptr) {            // K-smoothing: stored back centred
              center_block(T, b, wv);
              lds_blk[(2 * slot) * kResThreads + threadIdx.x] = u32x4{wv[0], wv[1], wv[2], wv[3]};
              lds_blk[(2 * slot + 1) * kResThreads + threadIdx.x] = u32x4{wv[4], wv[5], wv[6], wv[7]};
            }
          }
          const uint32_t am = absmax16(wv);
          ml[j] = ml[j] > am ? ml[j] : am;
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint32_t m = ms > ml[j] ? ms : ml[j];
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const uint32_t am = absmax16(w[j][i]);
      m = m > am ? m : am;
    }
    const uint32_t bmax = block_max_u32<kResThreads>(m, red[j]);
    // thread 0 publishes slot k; thread i >= 1 stamps slot k + i·nwg (1024
    // threads cover every slot above the grid)
    const int64_t s = k + (int64_t)threadIdx.x * nwg;
    if (s < kResidentSlots)
      __hip_atomic_store(args.t[j].slots + s, (epoch << 16) | (threadIdx.x == 0 ? bmax : 0u),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // poll: thread p < nwg watches slot p of every tensor
  const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + wait_ticks;
  uint32_t a[NJ], pending = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    a[j] = 0;
    if ((int)threadIdx.x < nwg) pending |= 1u << j;
  }
  while (true) {
    uint64_t sw[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      sw[j] = (pending >> j) & 1u ? load_slot(args.t[j].slots + threadIdx.x) : 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (((pending >> j) & 1u) && (sw[j] >> 16) == epoch) {
        a[j] = (uint32_t)(sw[j] & 0xFFFFu);
        pending &= ~(1u << j);
      }
    if (__syncthreads_and(pending == 0)) break;
    if (__syncthreads_or(__builtin_amdgcn_s_memrealtime() > deadline)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  // Fold the slots seen and note the unseen ones, behind one barrier.  Every
  // thread left the poll loop through a barrier, after its last read of red[]
  // in the publish step, so red[] can be written again without one.
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint32_t m = wave_max_u32(a[j]);
    const uint64_t mb = __ballot(((pending >> j) & 1u) != 0u);
    if (lane == 0) {
      red[j][wv] = m;
      miss[j][wv] = mb;
    }
  }
  __syncthreads();
  uint32_t A[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    uint32_t r = red[j][0];
    uint64_t any = miss[j][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      r = r > red[j][w] ? r : red[j][w];
      any |= miss[j][w];
    }
    if (any != 0) {        // the wait expired: read the missing shares directly
      uint32_t md = 0;
      for (int w = 0; w < NW; ++w)
        for (uint64_t mb = miss[j][w]; mb != 0; mb &= mb - 1) {
          const uint32_t v = share_max<STREAM, NJ == 2>(args.t[j], 64 * w + __builtin_ctzll(mb), u, nwg);
          md = md > v ? md : v;
        }
      const uint32_t rd = block_max_u32<kResThreads>(md, red2[j]);
      r = r > rd ? r : rd;
    }
    A[j] = r;
  }

#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const QuantTensor &T = args.t[j];
    const uint32_t Abits = A[j];
    const float g = (Abits == 0) ? 1.0f : bf16_bits_to_f32(Abits) / kGlobalDivisor;
    const BlockScaler b6(g, kE2M1Max), b4(g, 4.0f);
    if (k == 0 && threadIdx.x == 0) {
      *T.gscale = g;
      if (j == 0 && args.mark.chunk_start != nullptr) {
        args.mark.chunk_start[args.mark.index] = args.mark.value;
        if (args.mark.index == 1) args.mark.chunk_start[0] = 0;
      }
    }
    u32x2 *codes = reinterpret_cast<u32x2 *>(T.codes);
    uint8_t *scales = reinterpret_cast<uint8_t *>(T.scales);
#pragma unroll
    for (int i = 0; i < UMAX; ++i) {
      const int64_t b = ((int64_t)k * u + i) * kResThreads + threadIdx.x;
      uint32_t lo, hi;
      const uint32_t S = encode_any<ADAPT>(w[j][i], absmax16(w[j][i]), b6, b4, lo, hi);
      if (i < u && b < 2 * T.units) {
        codes[b] = u32x2{lo, hi};
        scales[b] = (uint8_t)S;
      }
    }
    if constexpr (LDSRES) {
      const int64_t nb = 2 * T.units;
      // the thread index made opaque, so these indices are recomputed here
      // instead of being kept in registers (spilled) since the prologue
      uint32_t tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
#pragma unroll
      for (int i = 0; i < ULDS; ++i) {
        const int64_t b = ((int64_t)k * u + UMAX + i) * kResThreads + tid;
        const int slot = j * ULDS + i;
        const u32x4 lo4 = lds_blk[(2 * slot) * kResThreads + tid];
        const u32x4 hi4 = lds_blk[(2 * slot + 1) * kResThreads + tid];
        const uint32_t wv[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
        uint32_t lo, hi;
        const uint32_t S = encode_any<ADAPT>(wv, absmax16(wv), b6, b4, lo, hi);
        if (UMAX + i < u && b < nb) {
          codes[b] = u32x2{lo, hi};
          scales[b] = (uint8_t)S;
        }
      }
    }
    if constexpr (STREAM) {
      const int64_t nb = 2 * T.units, cstride = (int64_t)nwg * kResThreads;
      const int64_t chunk0 = cstride * u + (int64_t)k * kResThreads + threadIdx.x;
      for (int64_t b0 = chunk0; b0 < nb; b0 += kStreamU * cstride) {
        uint32_t v[kStreamU][8];
#pragma unroll
        for (int i = 0; i < kStreamU; ++i) {
          const int64_t b = b0 + i * cstride;
          if (b < nb) {
            load_block<false>(T, b, v[i]);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = 0u;
          }
        }
#pragma unroll
        for (int i = 0; i < kStreamU; ++i) {
          const int64_t b = b0 + i * cstride;
          uint32_t lo, hi;
          const uint32_t S = encode_any<ADAPT>(v[i], absmax16(v[i]), b6, b4, lo, hi);
          if (b < nb) {
            codes[b] = u32x2{lo, hi};
            scales[b] = (uint8_t)S;
          }
        }
      }
    }
  }
}

// Resident-launch limits of a device: CU count and whether each kernel
// instance fits one workgroup per CU.
struct ResidentLimits {
  int cus = 0;
  bool fits[2][2][4] = {};                // [ADAPT][NJ - 1][log2 UMAX]
  bool fits_stream[2] = {};               // [ADAPT]: the STREAM kernel (one tensor, UMAX 8)
  bool fits_pair[2] = {};                 // [ADAPT]: the PAIRLDS kernel (K/V, UMAX 4 + LDS)
};

template <int NJ, int UMAX, bool ADAPT, bool STREAM = false, bool PAIRLDS = false>
static const void *resident_fn() {
  return reinterpret_cast<const void *>(&k_quant_resident<NJ, UMAX, ADAPT, STREAM, PAIRLDS>);
}

static const ResidentLimits &resident_limits() {
  static std::mutex mu;
  static ResidentLimits table[64];
  static bool filled[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!filled[dev]) {
    ResidentLimits &r = table[dev];
    if (hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) r.cus = 0;
    const void *fns[2][2][4] = {
        {{resident_fn<1, 1, false>(), resident_fn<1, 2, false>(), resident_fn<1, 4, false>(),
          resident_fn<1, 8, false>()},
         {resident_fn<2, 1, false>(), resident_fn<2, 2, false>(), resident_fn<2, 4, false>(), nullptr}},
        {{resident_fn<1, 1, true>(), resident_fn<1, 2, true>(), resident_fn<1, 4, true>(),
          resident_fn<1, 8, true>()},
         {resident_fn<2, 1, true>(), resident_fn<2, 2, true>(), resident_fn<2, 4, true>(), nullptr}}};
    for (int a = 0; a < 2; ++a)
      for (int j = 0; j < 2; ++j)
        for (int i = 0; i < 4; ++i) {
          int n = 0;
          r.fits[a][j][i] = fns[a][j][i] != nullptr &&
                            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fns[a][j][i], kResThreads,
                                                                         0) == hipSuccess &&
                            n >= 1;
        }
    const void *sfns[2] = {resident_fn<1, 8, false, true>(), resident_fn<1, 8, true, true>()};
    for (int a = 0; a < 2; ++a) {
      int n = 0;
      r.fits_stream[a] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, sfns[a], kResThreads, 0) ==
                             hipSuccess && n >= 1;
    }
    const void *pfns[2] = {resident_fn<2, 4, false, false, true>(), resident_fn<2, 4, true, false, true>()};
    for (int a = 0; a < 2; ++a) {
      int n = 0;
      r.fits_pair[a] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, pfns[a], kResThreads, 0) ==
                           hipSuccess && n >= 1;
    }
    filled[dev] = true;
  }
  return table[dev];
}

// Launches the resident quantiser (at most one workgroup per CU) when the
// tensors fit in its registers; returns false (nothing launched) otherwise.
template <bool ADAPT>
static bool launch_resident(QuantArgs &a, int njobs, int64_t max_units, hipStream_t stream,
                            hipError_t *err) {
  const ResidentLimits &lim = resident_limits();
  if (lim.cus < 1) return false;
  const int64_t nb = 2 * max_units;                         // 16-element blocks per tensor
  int64_t nwg = (nb + kResThreads - 1) / kResThreads;
  if (nwg > lim.cus) nwg = lim.cus;
  if (nwg > kResidentSlots) nwg = kResidentSlots;       // one polling thread per slot
  const int64_t u = (nb + nwg * kResThreads - 1) / (nwg * kResThreads);
  int li = 0;
  while (li < 4 && (1 << li) < u) ++li;
  const uint64_t wt = g_wait_ticks.load();
  if (njobs == 2 && u > 4 && u <= 4 + kLdsBlocks / 2) {
    // a K/V pair beyond the registers: 4 blocks per thread per tensor in
    // registers and 2 in LDS (an 8-frame chunk of 7040 tokens fits)
    if (!lim.fits_pair[ADAPT]) return false;
    hipLaunchKernelGGL((k_quant_resident<2, 4, ADAPT, false, true>), dim3((unsigned)nwg), dim3(kResThreads),
                       0, stream, a, (int)u, wt);
    *err = hipGetLastError();
    return true;
  }
  if (li == 4) {
    // more than the grid's registers hold: keep 8 blocks per thread resident
    // in registers and kLdsBlocks in LDS, and stream the rest (one tensor
    // only; else the two-pass kernels)
    if (njobs != 1 || !lim.fits_stream[ADAPT] || a.t[0].center != nullptr) return false;   // LDS blocks are not centred
    // the fewest blocks per thread that cover the tensor (every workgroup
    // busy), at most what registers and LDS hold
    const int us = (int)(u < 8 + kLdsBlocks ? u : 8 + kLdsBlocks);
    hipLaunchKernelGGL((k_quant_resident<1, 8, ADAPT, true>), dim3((unsigned)nwg), dim3(kResThreads), 0,
                       stream, a, us, wt);
    *err = hipGetLastError();
    return true;
  }
  if (!lim.fits[ADAPT][njobs - 1][li]) return false;
  const dim3 grid((unsigned)nwg), block(kResThreads);
  const int ui = (int)u;
  if (njobs == 1) {
    switch (li) {
      case 0: hipLaunchKernelGGL((k_quant_resident<1, 1, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
      case 1: hipLaunchKernelGGL((k_quant_resident<1, 2, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
      case 2: hipLaunchKernelGGL((k_quant_resident<1, 4, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
      default: hipLaunchKernelGGL((k_quant_resident<1, 8, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
    }
  } else {
    switch (li) {
      case 0: hipLaunchKernelGGL((k_quant_resident<2, 1, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
      case 1: hipLaunchKernelGGL((k_quant_resident<2, 2, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
      default: hipLaunchKernelGGL((k_quant_resident<2, 4, ADAPT>), grid, block, 0, stream, a, ui, wt); break;
    }
  }
  *err = hipGetLastError();
  return true;
}

// ---------------------------------------------------------------------------

static int amax_blocks(int64_t units) {
  const int64_t per = (int64_t)kThreads * kTwoPassU;            // blocks per workgroup round
  int64_t b = (2 * units + per - 1) / per;
  if (b < 1) b = 1;
  if (b > kAmaxBlocks) b = kAmaxBlocks;
  return (int)b;
}

static int encode_blocks(int64_t units) {
  const int64_t per = (int64_t)kThreads * kTwoPassU;
  int64_t b = (2 * units + per - 1) / per;
  if (b > 4096) b = 4096;
  if (b < 1) b = 1;
  return (int)b;
}

uint64_t set_resident_wait_ticks(uint64_t ticks) { return g_wait_ticks.exchange(ticks); }

hipError_t launch_encode_from_partials(const QuantJob &job, const uint32_t *maxima, int64_t nparts,
                                       hipStream_t stream) {
  QuantArgs a{};
  a.t[0].x = job.x;
  a.t[0].codes = job.codes;
  a.t[0].scales = reinterpret_cast<uint16_t *>(job.scales);
  a.t[0].gscale = job.gscale;
  a.t[0].partials = const_cast<uint32_t *>(maxima);
  a.t[0].units = job.rows * (job.cols / 32);
  a.t[0].units_per_row = (uint32_t)(job.cols / 32);
  a.t[0].ld = job.ld;
  a.t[0].center = job.center;
  if (nparts < 1 || nparts > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_encode<false>, dim3(encode_blocks(a.t[0].units), 1), dim3(kThreads), 0, stream, a,
                     (int)nparts);
  return hipGetLastError();
}

hipError_t launch_encode2_from_partials(const QuantJob (&jobs)[2], const uint32_t *const (&maxima)[2],
                                        int64_t nparts, const ChunkMark &mark, bool adaptive46,
                                        hipStream_t stream) {
  QuantArgs a{};
  a.mark = mark;
  int64_t max_units = 0;
  for (int i = 0; i < 2; ++i) {
    a.t[i].x = jobs[i].x;
    a.t[i].codes = jobs[i].codes;
    a.t[i].scales = reinterpret_cast<uint16_t *>(jobs[i].scales);
    a.t[i].gscale = jobs[i].gscale;
    a.t[i].partials = const_cast<uint32_t *>(maxima[i]);
    a.t[i].units = jobs[i].rows * (jobs[i].cols / 32);
    a.t[i].units_per_row = (uint32_t)(jobs[i].cols / 32);
    a.t[i].ld = jobs[i].ld;
    a.t[i].center = jobs[i].center;
    if (a.t[i].units > max_units) max_units = a.t[i].units;
  }
  if (nparts < 1 || nparts > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(encode_blocks(max_units), 2);
  if (adaptive46)
    hipLaunchKernelGGL(k_encode<true>, grid, dim3(kThreads), 0, stream, a, (int)nparts);
  else
    hipLaunchKernelGGL(k_encode<false>, grid, dim3(kThreads), 0, stream, a, (int)nparts);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantJob *jobs, int njobs, hipStream_t stream,
                           const ChunkMark *mark, bool adaptive46, bool blocks2d) {
  QuantArgs a{};
  if (mark) a.mark = *mark;
  int64_t max_units = 0;
  for (int i = 0; i < njobs; ++i) {
    a.t[i].x = jobs[i].x;
    a.t[i].codes = jobs[i].codes;
    a.t[i].scales = reinterpret_cast<uint16_t *>(jobs[i].scales);
    a.t[i].gscale = jobs[i].gscale;
    uint8_t *scratch = static_cast<uint8_t *>(jobs[i].scratch);
    a.t[i].slots = reinterpret_cast<uint64_t *>(scratch);
    a.t[i].partials = reinterpret_cast<uint32_t *>(scratch + kPartialsOffset);
    a.t[i].units = jobs[i].rows * (jobs[i].cols / 32);
    a.t[i].units_per_row = (uint32_t)(jobs[i].cols / 32);
    a.t[i].ld = jobs[i].ld;
    a.t[i].center = jobs[i].center;
    if (a.t[i].units > max_units) max_units = a.t[i].units;
  }
  // centres are carried by the kernels that take K/V pairs only
  if (njobs != 2 && a.t[0].center != nullptr) return hipErrorInvalidValue;
  if (blocks2d && (a.t[0].center != nullptr || (njobs == 2 && a.t[1].center != nullptr))) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (blocks2d) {             // two passes: tensor amax, then one thread per 16x16 tile
    if (njobs != 1 || adaptive46 || mark != nullptr) return hipErrorInvalidValue;
    const int nparts = amax_blocks(a.t[0].units);
    hipLaunchKernelGGL(k_amax, dim3(nparts, 1), dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t tiles = (jobs[0].rows + 15) / 16 * (jobs[0].cols / 16);
    const int64_t blocks = (tiles + kThreads - 1) / kThreads;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_encode_2d, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, nparts,
                       jobs[0].rows);
    return hipGetLastError();
  }
  if (adaptive46 ? launch_resident<true>(a, njobs, max_units, stream, &e)
                 : launch_resident<false>(a, njobs, max_units, stream, &e))
    return e;
  // Both tensors of a pair use the same grid; a tensor with fewer units simply
  // leaves some threads idle.
  const int nparts = amax_blocks(max_units);
  hipLaunchKernelGGL(k_amax, dim3(nparts, njobs), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (adaptive46)
    hipLaunchKernelGGL(k_encode<true>, dim3(encode_blocks(max_units), njobs), dim3(kThreads), 0, stream,
                       a, nparts);
  else
    hipLaunchKernelGGL(k_encode<false>, dim3(encode_blocks(max_units), njobs), dim3(kThreads), 0, stream,
                       a, nparts);
  return hipGetLastError();
}

}  // namespace nvfp4
