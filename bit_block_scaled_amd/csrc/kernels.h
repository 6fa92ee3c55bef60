// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Upper bound on the number of amax partials a two-pass quantisation writes.
constexpr int kAmaxBlocks = 1024;
// Slots of a resident (single-pass) quantisation: one 64-bit word per
// workgroup plus the published result at index kResidentSlots.
constexpr int kResidentSlots = 4096;
// Scratch bytes per quantised tensor (covers both uses; a multiple of 256).
constexpr size_t kQuantScratchBytes = 8 * (size_t(kResidentSlots) + 32);

// One tensor to quantise: `rows` rows of `cols` bf16 values (cols a multiple of
// 32), row r starting at x + r·ld, into dense codes (rows·cols/2 bytes),
// scales (rows·cols/16 bytes) and *gscale, using `partials`
// (kQuantScratchBytes, 8-byte aligned) as scratch.  A dense matrix may be passed as one row.
struct QuantJob {
  const uint16_t *x;
  uint8_t *codes;
  uint8_t *scales;
  float *gscale;
  uint32_t *partials;
  int64_t rows, cols, ld;
};

// KV-cache bookkeeping written by the encode launch of an append:
// chunk_start[index] = value (and chunk_start[0] = 0 when index == 1).
struct ChunkMark {
  int64_t *chunk_start;
  int64_t index;
  int64_t value;
};

// Encodes one tensor in a single pass when its |x| maximum is already known as
// the largest of `nparts` 15-bit bf16 magnitude patterns at job.partials (the
// per-tile maxima a GEMM epilogue wrote): the same bytes as launch_quantize.
hipError_t launch_encode_from_partials(const QuantJob &job, int64_t nparts, hipStream_t stream);

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
  // outputs (the 15-bit pattern of the bf16 result) to tile_amax[tile]; the
  // array has gemm_tile_count(...) entries
  uint32_t *tile_amax = nullptr;
};

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream);

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
};

hipError_t launch_kv_dequant(const KvDequantArgs &a, hipStream_t stream);

}  // namespace nvfp4
