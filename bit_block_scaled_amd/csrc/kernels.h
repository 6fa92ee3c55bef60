// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Upper bound on the number of amax partials a two-pass quantisation writes.
constexpr int kAmaxBlocks = 1024;
// Most workgroups of a resident (single-pass) quantisation: one 64-bit slot
// each, every slot polled by one thread of a 1024-thread workgroup.
constexpr int kResidentSlots = 1024;
// Scratch of one quantised tensor, 256-byte aligned, all zero before its first
// use (the library keeps it valid from one call to the next):
//   [0, kPartialsOffset)             resident slots, one (epoch, max) word per
//                                    slot; a resident call leaves all of them
//                                    with its epoch
//   [kPartialsOffset, kQuantScratchBytes)  partial maxima of the two-pass kernels
constexpr size_t kPartialsOffset = 8 * size_t(kResidentSlots);
constexpr size_t kQuantScratchBytes = kPartialsOffset + 4 * size_t(kAmaxBlocks);
static_assert(kQuantScratchBytes % 256 == 0, "scratch regions stay 256-byte aligned");

// One tensor to quantise: `rows` rows of `cols` bf16 values (cols a multiple of
// 32), row r starting at x + r·ld, into dense codes (rows·cols/2 bytes),
// scales (rows·cols/16 bytes) and *gscale, using `scratch`
// (kQuantScratchBytes, laid out as above).  A dense matrix may be passed as one row.
struct QuantJob {
  const uint16_t *x;
  uint8_t *codes;
  uint8_t *scales;
  float *gscale;
  void *scratch;
  int64_t rows, cols, ld;
  // K-smoothing: bf16 [cols] channel centres subtracted from every row as it
  // is loaded, bf16_rne(fl32(x − center)); null for none.  Used by the KV
  // append (two tensors per launch).
  const uint16_t *center = nullptr;
};

// KV-cache bookkeeping written by the encode launch of an append:
// chunk_start[index] = value (and chunk_start[0] = 0 when index == 1).
struct ChunkMark {
  int64_t *chunk_start;
  int64_t index;
  int64_t value;
};

// Encodes one tensor in a single pass when its |x| maximum is already known as
// the largest of `nparts` 15-bit bf16 magnitude patterns at `maxima` (the
// per-tile maxima a GEMM epilogue wrote): the same bytes as launch_quantize.
// job.scratch is not used.
hipError_t launch_encode_from_partials(const QuantJob &job, const uint32_t *maxima, int64_t nparts,
                                       hipStream_t stream);

// The same for two tensors in one launch (a KV append: K and V), each with its
// own nparts maxima, with the KV-cache bookkeeping `mark` and optionally the
// adaptive {4, 6} block scales.
hipError_t launch_encode2_from_partials(const QuantJob (&jobs)[2], const uint32_t *const (&maxima)[2],
                                        int64_t nparts, const ChunkMark &mark, bool adaptive46,
                                        hipStream_t stream);

// Bounded wait of the single-launch quantiser for the other workgroups'
// maxima, in ticks of the 100 MHz real-time counter; returns the previous
// value.  The results do not depend on it (a workgroup whose wait expires
// computes the tensor maximum itself).
uint64_t set_resident_wait_ticks(uint64_t ticks);

// Quantises one or two tensors (njobs in {1, 2}) on `stream`: one launch when
// the grid fits on the device at once, else two launches.
// adaptive46 selects the adaptive {4, 6} block scales; blocks2d the 16x16
// two-dimensional blocks (one tensor, no mark, not with adaptive46: two
// launches).
hipError_t launch_quantize(const QuantJob *jobs, int njobs, hipStream_t stream,
                           const ChunkMark *mark = nullptr, bool adaptive46 = false,
                           bool blocks2d = false);

struct GemmArgs {
  const uint8_t *Aq;
  const uint8_t *As;
  const float *Ag;
  const uint8_t *Wq;
  const uint8_t *Ws;
  const float *Wg;
  const uint16_t *bias;
  uint16_t *C;
  int64_t M, N, K;
  uint32_t flags;
  // optional: every workgroup tile writes the largest magnitude of its stored
  // outputs (the 15-bit pattern of the bf16 result) to
  // tile_amax[tn · tiles_m + tm] for the tile in tile row tm, tile column tn
  // (column-major, so the tiles of a range of output columns are
  // contiguous); the array has gemm_tile_count(...) entries
  uint32_t *tile_amax = nullptr;
};

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);

// Workgroup tile (bm x bn) launch_gemm uses for these arguments.
void gemm_tile_of(const GemmArgs &a, int *bm, int *bn);

// Number of workgroup tiles launch_gemm uses for these arguments.
int64_t gemm_tile_count(const GemmArgs &a);

// Tile shape chosen for a problem (exposed for the benchmark's reporting).
void gemm_tile_for(int64_t M, int64_t N, int64_t K, int *bm, int *bn);

struct KvDequantArgs {
  const uint8_t *codes[2];
  const uint8_t *scales[2];
  uint16_t *out[2];
  const float *gscale;          // [chunks, 2]
  const int64_t *chunk_start;   // [chunks + 1]
  int64_t n_chunks;
  int64_t t0, t1;
  int64_t elems_per_token;      // heads · head_dim (multiple of 32)
  const uint16_t *kcenter;      // K-smoothing: bf16 [chunks, elems_per_token] centres, or null
};

hipError_t launch_kv_dequant(const KvDequantArgs &a, hipStream_t stream);

// K-smoothing of one appended chunk: keys k [T, e] bf16 (token t at k + t·ld,
// e and ld multiples of 8, 16-byte aligned), the channel centres written to
// center [e] (bf16; the quantiser subtracts them as it loads K, see
// QuantJob::center).  partials holds smooth_partial_count(T, e) 64-bit
// integers, written before they are read.
struct SmoothArgs {
  const uint16_t *k;
  int64_t T, e, ld;
  int64_t *partials;
  uint16_t *center;
};
int64_t smooth_partial_count(int64_t T, int64_t e);
hipError_t launch_kv_smooth(const SmoothArgs &a, hipStream_t stream);

// Attention of bf16 queries over keys/values from the NVFP4 cache (or, for the
// bf16 twin, from bf16 K/V tensors).  head_dim is 128.  Keys are the tokens of
// up to kAttnMaxRanges disjoint ranges, concatenated ("virtual keys"
// 0 .. Tk-1); the workgroups split them into nsplit parts of keys_per_split
// keys (a multiple of 64); with nsplit > 1, part_o [nsplit][Tq][heads][128]
// and part_ml [nsplit][Tq][heads][2] hold the partial results.
constexpr int kAttnMaxRanges = 4;
struct AttnArgs {
  const uint16_t *q;            // bf16, query t head h at q + t·ldq + 128·h
  int64_t ldq;
  uint16_t *o;                  // bf16 output, same layout with ldo
  int64_t ldo;
  int64_t Tq, heads;
  const uint8_t *kc, *ks, *vc, *vs;     // NVFP4 cache codes / scales
  const float *gscale;
  const int64_t *chunk_start;
  int64_t n_chunks;
  const uint16_t *kb, *vb;              // bf16 twin: token t head h at kb + t·ldkv + 128·h
  int64_t ldkv;
  int64_t kv_tokens;                    // tokens addressable in the K/V buffers (< 2^24,
                                        // and each buffer below 2^31 bytes)
  int64_t range_lo[kAttnMaxRanges], range_len[kAttnMaxRanges];
  int n_ranges;
  int64_t Tk;
  float qk_scale;               // scale · log2(e)
  const uint16_t *kcenter;      // K-smoothing: bf16 [chunks, heads·128] centres, or null
  int nsplit;
  int64_t keys_per_split;
  float *part_o, *part_ml;
};
int64_t attention_splits(int64_t Tq, int64_t heads, int64_t Tk);
int64_t attention_keys_per_split(int64_t Tk, int64_t nsplit);
hipError_t launch_attention(const AttnArgs &a, bool bf16, hipStream_t stream);

// Weight-gradient operand: x [T, N] bf16 (token t at x + t·ld, T a multiple of
// 32, ld a multiple of 8), transformed per group of 16 tokens by
// H16·diag(s)/4 (s_k = −1 where bit k of sign_mask is set) and quantised as
// its transpose [N, T]: codes [N, T/2], scales [N, T/16], *gscale.  partials
// holds kRhtMaxParts words, written before they are read (no initialisation).
constexpr int kRhtMaxParts = 2048;
struct RhtArgs {
  const uint16_t *x;
  int64_t T, N, ld;
  uint32_t sign_mask;
  uint8_t *codes, *scales;
  float *gscale;
  uint32_t *partials;
};
int64_t rht_tiles(int64_t T, int64_t N);
hipError_t launch_quantize_rht(const RhtArgs &a, hipStream_t stream);

}  // namespace nvfp4
