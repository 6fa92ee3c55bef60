// NVFP4 GEMM, host side: the workgroup-tile choice and the launch of the
// chosen tile's kernels (the kernel itself is in gemm_kernel.h).
#include <atomic>

#include "gemm_kernel.h"

namespace nvfp4 {

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
    // (256x256 runs one tile per workgroup, without the persistent prefetch;
    // measured on the DiT shapes this costs nothing measurable, so no penalty)
    const double cost = rounds * (double)bm * bn * (1.0 + 0.25 * (1.0 / c.wm + 1.0 / c.wn));
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

static int device_cus() {
  static std::atomic<int> cached[64];      // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static TileChoice tile_of(const GemmArgs &a) {
  static const TileChoice by_flag[] = {{0, 0}, {4, 4}, {4, 3}, {3, 4}, {4, 2}, {2, 4}, {2, 2}};
  const uint32_t tf = (a.flags & NVFP4_TILE_MASK) >> 8;
  return tf ? by_flag[tf] : choose_tile(a.M, a.N);
}

void gemm_tile_of(const GemmArgs &a, int *bm, int *bn) {
  const TileChoice c = tile_of(a);
  *bm = 64 * c.wm;
  *bn = 64 * c.wn;
}

int64_t gemm_tile_count(const GemmArgs &a) {
  const TileChoice c = tile_of(a);
  const int64_t bm = 64 * c.wm, bn = 64 * c.wn;
  return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t stream) {
  const TileChoice c = tile_of(a);
  const int cus = device_cus();
  if (c.wm == 4 && c.wn == 4) return launch_gemm_4x4(a, stream, cus);
  if (c.wm == 4 && c.wn == 3) return launch_gemm_4x3(a, stream, cus);
  if (c.wm == 3 && c.wn == 4) return launch_gemm_3x4(a, stream, cus);
  if (c.wm == 4 && c.wn == 2) return launch_gemm_4x2(a, stream, cus);
  if (c.wm == 2 && c.wn == 4) return launch_gemm_2x4(a, stream, cus);
  return launch_gemm_2x2(a, stream, cus);
}

}  // namespace nvfp4
