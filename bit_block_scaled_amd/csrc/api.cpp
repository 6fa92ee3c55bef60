// C ABI of the NVFP4 library: argument validation, workspace layout and
// kernel launches.  Every entry point is declared (with its contract) in
// include/nvfp4.h.
#include <nvfp4.h>
#include <nvfp4_testing.h>

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string.h>

#include <atomic>
#include <string>

#include "kernels.h"

namespace {

// The calling thread's last error message.  A plain character array: it has
// no destructor, so nothing of this library runs when a thread or the process
// exits.
thread_local char g_last_error[512];

int fail(int status, const std::string &msg) {
  const size_t n = msg.size() < sizeof(g_last_error) - 1 ? msg.size() : sizeof(g_last_error) - 1;
  memcpy(g_last_error, msg.data(), n);
  g_last_error[n] = '\0';
  return status;
}

bool aligned(const void *p, size_t a = NVFP4_ALIGN) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxElements = int64_t(1) << 36;   // keeps unit indices below 2^31
constexpr size_t kQuantWs = nvfp4::kQuantScratchBytes;
// Every workspace starts with the same head: the scratch of two quantised
// tensors (regions 0 and 1), written only by the quantiser (its slots and its
// two-pass partial maxima); every other buffer of a workspace lies after it.
// So one zeroed buffer can serve calls of any kind and size: no call writes
// data where another keeps quantiser slots.
constexpr size_t kWsHead = 2 * kQuantWs;

int check_mk(int64_t M, int64_t K, const char *who) {
  if (M < 1) return fail(NVFP4_EINVAL, std::string(who) + ": M must be >= 1");
  if (K < 32 || K % 32) return fail(NVFP4_EINVAL, std::string(who) + ": K must be a positive multiple of 32");
  if (M > kMaxElements / K) return fail(NVFP4_EINVAL, std::string(who) + ": M*K too large");
  return NVFP4_OK;
}

int check_ptr(const void *p, const char *name, size_t align = NVFP4_ALIGN) {
  if (p == nullptr) return fail(NVFP4_EINVAL, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(NVFP4_EINVAL, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return NVFP4_OK;
}

int hip_status(hipError_t e, const char *who) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_EHIP, std::string(who) + ": " + hipGetErrorString(e));
}

// Testing hook state (nvfp4_testing_set_launch_events): events still to be
// recorded, one after each launch step, on the step's stream.
std::atomic<void *const *> g_events{nullptr};
std::atomic<int> g_events_left{0}, g_events_next{0};

// Status of a launch step on `st`; after a successful one, records the next
// pending testing event there (if any).
int launched(hipError_t e, hipStream_t st, const char *who) {
  const int s = hip_status(e, who);
  if (s == NVFP4_OK && g_events_left.load(std::memory_order_relaxed) > 0) {
    void *const *ev = g_events.load(std::memory_order_relaxed);
    const int i = g_events_next.fetch_add(1, std::memory_order_relaxed);
    g_events_left.fetch_sub(1, std::memory_order_relaxed);
    if (ev != nullptr) return hip_status(hipEventRecord(static_cast<hipEvent_t>(ev[i]), st), who);
  }
  return s;
}

// nvfp4_linear workspace: [head (quantiser scratch of x in region 0) | codes | scales | gscale]
struct LinearWs {
  size_t partials, codes, scales, gscale, total;
};

LinearWs linear_ws(int64_t M, int64_t K) {
  LinearWs w;
  const size_t n = size_t(M) * size_t(K);
  w.partials = 0;
  w.codes = kWsHead;
  w.scales = round_up(w.codes + n / 2, 256);
  w.gscale = round_up(w.scales + n / 16, 256);
  w.total = round_up(w.gscale + sizeof(float), 256);
  return w;
}

int check_gemm_args(const uint8_t *Aq, const uint8_t *As, const float *Ag, const uint8_t *Wq,
                    const uint8_t *Ws, const float *Wg, const uint16_t *bias, const uint16_t *C,
                    int64_t M, int64_t N, int64_t K, uint32_t flags, bool check_a) {
  int s;
  if ((s = check_mk(M, K, "gemm"))) return s;
  if (N < 1) return fail(NVFP4_EINVAL, "gemm: N must be >= 1");
  if (N > kMaxElements / K || M > kMaxElements / N) return fail(NVFP4_EINVAL, "gemm: problem too large");
  if (K > (int64_t(1) << 24)) return fail(NVFP4_EINVAL, "gemm: K must be <= 2^24");
  if (flags & ~uint32_t(NVFP4_EPI_GELU_TANH | NVFP4_TILE_MASK))
    return fail(NVFP4_EINVAL, "gemm: unknown flag bits");
  if ((flags & NVFP4_TILE_MASK) > NVFP4_TILE_128x128) return fail(NVFP4_EINVAL, "gemm: unknown tile flag");
  if (check_a) {
    if ((s = check_ptr(Aq, "Aq"))) return s;
    if ((s = check_ptr(As, "As"))) return s;
    if ((s = check_ptr(Ag, "Ag", 4))) return s;
  }
  if ((s = check_ptr(Wq, "Wq"))) return s;
  if ((s = check_ptr(Ws, "Ws"))) return s;
  if ((s = check_ptr(Wg, "Wg", 4))) return s;
  if (bias && !aligned(bias)) return fail(NVFP4_EINVAL, "bias is not 16-byte aligned");
  if ((s = check_ptr(C, "C"))) return s;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_quantize_workspace(int64_t M, int64_t K, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  int s = check_mk(M, K, "quantize_workspace");
  if (s) return s;
  *bytes = kQuantWs;
  return NVFP4_OK;
}

int nvfp4_quantize_ex(const uint16_t *x, int64_t M, int64_t K, uint32_t qflags, uint8_t *codes,
                      uint8_t *scales, float *gscale, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_mk(M, K, "quantize"))) return s;
  if (qflags & ~(NVFP4_Q_ADAPTIVE_4_6 | NVFP4_Q_BLOCK_2D)) return fail(NVFP4_EINVAL, "quantize: unknown flags");
  if ((qflags & NVFP4_Q_ADAPTIVE_4_6) && (qflags & NVFP4_Q_BLOCK_2D))
    return fail(NVFP4_EINVAL, "quantize: NVFP4_Q_ADAPTIVE_4_6 and NVFP4_Q_BLOCK_2D exclude each other");
  if ((s = check_ptr(x, "x"))) return s;
  if ((s = check_ptr(codes, "codes"))) return s;
  if ((s = check_ptr(scales, "scales"))) return s;
  if ((s = check_ptr(gscale, "gscale", 4))) return s;
  if (ws == nullptr || ws_bytes < kQuantWs) return fail(NVFP4_EWORKSPACE, "quantize: workspace too small");
  if ((s = check_ptr(ws, "ws"))) return s;
  nvfp4::QuantJob j{x, codes, scales, gscale, ws, M, K, K};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(nvfp4::launch_quantize(&j, 1, st, nullptr, (qflags & NVFP4_Q_ADAPTIVE_4_6) != 0,
                                         (qflags & NVFP4_Q_BLOCK_2D) != 0),
                  st, "quantize");
}

int nvfp4_quantize(const uint16_t *x, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales,
                   float *gscale, void *ws, size_t ws_bytes, void *stream) {
  return nvfp4_quantize_ex(x, M, K, 0u, codes, scales, gscale, ws, ws_bytes, stream);
}

int nvfp4_gemm(const uint8_t *Aq, const uint8_t *As, const float *Ag, const uint8_t *Wq,
               const uint8_t *Ws, const float *Wg, const uint16_t *bias, uint16_t *C, int64_t M,
               int64_t N, int64_t K, uint32_t flags, void *stream) {
  int s = check_gemm_args(Aq, As, Ag, Wq, Ws, Wg, bias, C, M, N, K, flags, true);
  if (s) return s;
  nvfp4::GemmArgs a{Aq, As, Ag, Wq, Ws, Wg, bias, C, M, N, K, flags};
  return launched(nvfp4::launch_gemm(a, static_cast<hipStream_t>(stream)), static_cast<hipStream_t>(stream),
                  "gemm");
}

int nvfp4_gemm_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn) {
  if (bm == nullptr || bn == nullptr) return fail(NVFP4_EINVAL, "gemm_tile: NULL output");
  if (M < 1 || N < 1 || K < 32 || K % 32) return fail(NVFP4_EINVAL, "gemm_tile: bad shape");
  nvfp4::gemm_tile_for(M, N, K, bm, bn);
  return NVFP4_OK;
}

int nvfp4_linear_workspace(int64_t M, int64_t K, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  int s = check_mk(M, K, "linear_workspace");
  if (s) return s;
  *bytes = linear_ws(M, K).total;
  return NVFP4_OK;
}

int nvfp4_linear(const uint16_t *x, const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                 const uint16_t *bias, uint16_t *C, int64_t M, int64_t N, int64_t K,
                 uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
  int s = check_gemm_args(nullptr, nullptr, nullptr, Wq, Ws, Wg, bias, C, M, N, K, flags, false);
  if (s) return s;
  if ((s = check_ptr(x, "x"))) return s;
  const LinearWs w = linear_ws(M, K);
  if (ws == nullptr || ws_bytes < w.total) return fail(NVFP4_EWORKSPACE, "linear: workspace too small");
  if ((s = check_ptr(ws, "ws"))) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  uint8_t *aq = base + w.codes;
  uint8_t *as = base + w.scales;
  float *ag = reinterpret_cast<float *>(base + w.gscale);
  hipStream_t st = static_cast<hipStream_t>(stream);
  nvfp4::QuantJob j{x, aq, as, ag, base + w.partials, M, K, K};
  if ((s = launched(nvfp4::launch_quantize(&j, 1, st), st, "linear/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, C, M, N, K, flags};
  return launched(nvfp4::launch_gemm(a, st), st, "linear/gemm");
}

// ---------------------------------------------------------------------------
// nvfp4_linear_noalloc: nvfp4_linear with its workspace in a file-scope device
// array, for callers that cannot allocate.  Layout (fixed, so the quantiser's
// call counter stays in place from one call to the next):
//   [0, kNoAllocMaxElements/2)            activation codes
//   [.., + kNoAllocMaxElements/16)        activation block scales
//   [.., + 256)                           activation tensor scale
//   [.., + kQuantScratchBytes)            quantiser scratch
// The array is zero when the code object is loaded, which is the state the
// quantiser scratch needs before its first use; the library keeps it valid.
constexpr size_t kNoAllocCodes = 0;
constexpr size_t kNoAllocScales = kNoAllocCodes + size_t(NVFP4_NOALLOC_MAX_ELEMENTS) / 2;
constexpr size_t kNoAllocGscale = kNoAllocScales + size_t(NVFP4_NOALLOC_MAX_ELEMENTS) / 16;
constexpr size_t kNoAllocQuant = kNoAllocGscale + 256;
constexpr size_t kNoAllocBytes = kNoAllocQuant + kQuantWs;
static_assert(kNoAllocScales % 256 == 0 && kNoAllocGscale % 256 == 0, "aligned regions");

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy of the array).  In host code the
// array's name stands for a host-side shadow, never for device memory.
static std::atomic<uintptr_t> g_scratch_addr[64];

static int noalloc_scratch(uint8_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "linear_noalloc: hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(NVFP4_EINVAL, "linear_noalloc: device index beyond 63");
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "linear_noalloc: hipGetSymbolAddress");
    if (p == nullptr) return fail(NVFP4_EHIP, "linear_noalloc: no device address for the scratch array");
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = reinterpret_cast<uint8_t *>(a);
  return NVFP4_OK;
}

// nvfp4_linear_q workspace: [linear workspace | tile maxima | H bf16 [M, N]]
struct LinearQWs {
  LinearWs lin;
  size_t slots, h, total;
  int64_t max_tiles;
};

static LinearQWs linear_q_ws(int64_t M, int64_t N, int64_t K) {
  LinearQWs w;
  w.lin = linear_ws(M, K);
  w.max_tiles = ((M + 127) / 128) * ((N + 127) / 128);   // the finest tiling the GEMM uses
  w.slots = w.lin.total;
  w.h = round_up(w.slots + size_t(w.max_tiles) * sizeof(uint32_t), 256);
  w.total = round_up(w.h + size_t(M) * size_t(N) * sizeof(uint16_t), 256);
  return w;
}

int nvfp4_linear_noalloc(const uint16_t *x, const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                         const uint16_t *bias, uint16_t *C, int64_t M, int64_t N, int64_t K,
                         uint32_t flags, void *stream) {
  int s = check_gemm_args(nullptr, nullptr, nullptr, Wq, Ws, Wg, bias, C, M, N, K, flags, false);
  if (s) return s;
  if ((s = check_ptr(x, "x"))) return s;
  if (M > NVFP4_NOALLOC_MAX_ELEMENTS / K)
    return fail(NVFP4_EINVAL, "linear_noalloc: M*K = " + std::to_string(M * K) +
                                  " exceeds the built-in workspace (NVFP4_NOALLOC_MAX_ELEMENTS = " +
                                  std::to_string(int64_t(NVFP4_NOALLOC_MAX_ELEMENTS)) + ")");
  uint8_t *base = nullptr;
  if ((s = noalloc_scratch(&base))) return s;
  uint8_t *aq = base + kNoAllocCodes;
  uint8_t *as = base + kNoAllocScales;
  float *ag = reinterpret_cast<float *>(base + kNoAllocGscale);
  hipStream_t st = static_cast<hipStream_t>(stream);
  nvfp4::QuantJob j{x, aq, as, ag, base + kNoAllocQuant, M, K, K};
  if ((s = launched(nvfp4::launch_quantize(&j, 1, st), st, "linear_noalloc/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, C, M, N, K, flags};
  return launched(nvfp4::launch_gemm(a, st), st, "linear_noalloc/gemm");
}

int nvfp4_linear_q_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  int s = check_mk(M, K, "linear_q_workspace");
  if (s) return s;
  if (N < 32 || N % 32) return fail(NVFP4_EINVAL, "linear_q_workspace: N must be a positive multiple of 32");
  if (N > kMaxElements / K || M > kMaxElements / N) return fail(NVFP4_EINVAL, "linear_q_workspace: problem too large");
  *bytes = linear_q_ws(M, N, K).total;
  return NVFP4_OK;
}

int nvfp4_linear_q(const uint16_t *x, const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                   const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint32_t flags, uint8_t *Hq,
                   uint8_t *Hs, float *Hg, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if (N < 32 || N % 32) return fail(NVFP4_EINVAL, "linear_q: N must be a positive multiple of 32");
  if ((s = check_mk(M, K, "linear_q"))) return s;
  if (N > kMaxElements / K || M > kMaxElements / N) return fail(NVFP4_EINVAL, "linear_q: problem too large");
  if ((s = check_ptr(ws, "ws"))) return s;
  const LinearQWs w = linear_q_ws(M, N, K);
  if (ws_bytes < w.total) return fail(NVFP4_EWORKSPACE, "linear_q: workspace too small");
  uint8_t *base = static_cast<uint8_t *>(ws);
  uint16_t *H = reinterpret_cast<uint16_t *>(base + w.h);
  if ((s = check_gemm_args(nullptr, nullptr, nullptr, Wq, Ws, Wg, bias, H, M, N, K, flags, false))) return s;
  if ((s = check_ptr(x, "x"))) return s;
  if ((s = check_ptr(Hq, "Hq"))) return s;
  if ((s = check_ptr(Hs, "Hs"))) return s;
  if ((s = check_ptr(Hg, "Hg", 4))) return s;
  uint8_t *aq = base + w.lin.codes;
  uint8_t *as = base + w.lin.scales;
  float *ag = reinterpret_cast<float *>(base + w.lin.gscale);
  uint32_t *slots = reinterpret_cast<uint32_t *>(base + w.slots);
  hipStream_t st = static_cast<hipStream_t>(stream);
  nvfp4::QuantJob jx{x, aq, as, ag, base + w.lin.partials, M, K, K};
  if ((s = launched(nvfp4::launch_quantize(&jx, 1, st), st, "linear_q/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, H, M, N, K, flags};
  a.tile_amax = slots;
  const int64_t tiles = nvfp4::gemm_tile_count(a);
  if (tiles > w.max_tiles) return fail(NVFP4_EHIP, "linear_q: internal tile count exceeds the workspace");
  if ((s = launched(nvfp4::launch_gemm(a, st), st, "linear_q/gemm"))) return s;
  nvfp4::QuantJob jh{H, Hq, Hs, Hg, nullptr, M, N, N};
  return launched(nvfp4::launch_encode_from_partials(jh, slots, tiles, st), st, "linear_q/encode");
}

int nvfp4_kv_init(nvfp4_kv_cache *c) {
  int s;
  if (c == nullptr) return fail(NVFP4_EINVAL, "kv_init: cache is NULL");
  if (c->capacity < 1 || c->heads < 1 || c->max_chunks < 1)
    return fail(NVFP4_EINVAL, "kv_init: capacity, heads and max_chunks must be >= 1");
  if (c->head_dim < 32 || c->head_dim % 32) return fail(NVFP4_EINVAL, "kv_init: head_dim must be a positive multiple of 32");
  if (c->capacity > kMaxElements / (c->heads * c->head_dim)) return fail(NVFP4_EINVAL, "kv_init: cache too large");
  if ((s = check_ptr(c->k_codes, "k_codes"))) return s;
  if ((s = check_ptr(c->v_codes, "v_codes"))) return s;
  if ((s = check_ptr(c->k_scales, "k_scales"))) return s;
  if ((s = check_ptr(c->v_scales, "v_scales"))) return s;
  if ((s = check_ptr(c->gscale, "gscale", 8))) return s;
  if ((s = check_ptr(c->chunk_start, "chunk_start", 8))) return s;
  if (c->k_center != nullptr && (s = check_ptr(c->k_center, "k_center"))) return s;
  if (c->k_center != nullptr && c->heads * c->head_dim > (int64_t(1) << 20))
    return fail(NVFP4_EINVAL, "kv_init: K-smoothing needs heads*head_dim <= 2^20");
  c->n_tokens = 0;
  c->n_chunks = 0;
  return NVFP4_OK;
}

int nvfp4_kv_append_workspace(int64_t T, int64_t heads, int64_t head_dim, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  if (T < 1 || heads < 1 || head_dim < 32 || head_dim % 32) return fail(NVFP4_EINVAL, "kv_append_workspace: bad geometry");
  *bytes = 2 * kQuantWs;
  return NVFP4_OK;
}

// Scratch a K-smoothed cache needs after an append's own workspace: the
// per-strip channel sums (no initialisation).
struct SmoothWs {
  size_t sums, total;
};
static SmoothWs smooth_ws(size_t base, int64_t T, int64_t e) {
  SmoothWs w;
  w.sums = round_up(base, 256);
  w.total = round_up(w.sums + size_t(nvfp4::smooth_partial_count(T, e)) * sizeof(int64_t), 256);
  return w;
}

int nvfp4_kv_smooth_workspace(int64_t T, int64_t heads, int64_t head_dim, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  if (T < 1 || heads < 1 || head_dim < 32 || head_dim % 32) return fail(NVFP4_EINVAL, "kv_smooth_workspace: bad geometry");
  if (heads * head_dim > (int64_t(1) << 20) || T > kMaxElements / (heads * head_dim))
    return fail(NVFP4_EINVAL, "kv_smooth_workspace: too large");
  *bytes = smooth_ws(0, T, heads * head_dim).total;
  return NVFP4_OK;
}

// Enqueues the channel centres of T keys (token stride ld) of the append
// about to be made as chunk c->n_chunks; returns that chunk's centre row,
// which the append's quantiser subtracts as it loads the keys.
static int enqueue_smoothing(const nvfp4_kv_cache *c, const uint16_t *K, int64_t T, int64_t ld,
                             uint8_t *ws, size_t base, hipStream_t st, const char *who,
                             const uint16_t **center) {
  const int64_t e = c->heads * c->head_dim;
  const SmoothWs w = smooth_ws(base, T, e);
  nvfp4::SmoothArgs sa{K, T, e, ld, reinterpret_cast<int64_t *>(ws + w.sums), c->k_center + c->n_chunks * e};
  *center = sa.center;
  return launched(nvfp4::launch_kv_smooth(sa, st), st, who);
}

static int check_cache(const nvfp4_kv_cache *c, const char *who) {
  if (c == nullptr) return fail(NVFP4_EINVAL, std::string(who) + ": cache is NULL");
  if (c->capacity < 1 || c->heads < 1 || c->head_dim < 32 || c->head_dim % 32 || c->max_chunks < 1 ||
      c->n_tokens < 0 || c->n_tokens > c->capacity || c->n_chunks < 0 || c->n_chunks > c->max_chunks ||
      !c->k_codes || !c->v_codes || !c->k_scales || !c->v_scales || !c->gscale || !c->chunk_start)
    return fail(NVFP4_EINVAL, std::string(who) + ": cache descriptor is not initialised");
  return NVFP4_OK;
}

int nvfp4_kv_append_ex(nvfp4_kv_cache *c, const uint16_t *K, const uint16_t *V, int64_t T,
                       int64_t ld, uint32_t qflags, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_cache(c, "kv_append"))) return s;
  if (qflags & ~NVFP4_Q_ADAPTIVE_4_6) return fail(NVFP4_EINVAL, "kv_append: unknown flags");
  if (T < 1) return fail(NVFP4_EINVAL, "kv_append: T must be >= 1");
  if (ld < c->heads * c->head_dim || ld % 8) return fail(NVFP4_EINVAL, "kv_append: ld must be >= heads*head_dim and a multiple of 8");
  if (T > kMaxElements / ld) return fail(NVFP4_EINVAL, "kv_append: T*ld too large");
  if ((s = check_ptr(K, "K"))) return s;
  if ((s = check_ptr(V, "V"))) return s;
  if (T > c->capacity - c->n_tokens) return fail(NVFP4_ECAPACITY, "kv_append: token capacity exceeded");
  if (c->n_chunks >= c->max_chunks) return fail(NVFP4_ECAPACITY, "kv_append: no chunk slot left");
  const int64_t e = c->heads * c->head_dim;           // elements per token
  const size_t need = c->k_center != nullptr ? smooth_ws(2 * kQuantWs, T, e).total : 2 * kQuantWs;
  if (ws == nullptr || ws_bytes < need) return fail(NVFP4_EWORKSPACE, "kv_append: workspace too small");
  if ((s = check_ptr(ws, "ws"))) return s;
  const int64_t off = c->n_tokens * e;
  uint8_t *parts = static_cast<uint8_t *>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t *center = nullptr;
  if (c->k_center != nullptr &&
      (s = enqueue_smoothing(c, K, T, ld, parts, 2 * kQuantWs, st, "kv_append/smooth", &center)))
    return s;
  nvfp4::QuantJob jobs[2] = {
      {K, c->k_codes + off / 2, c->k_scales + off / 16, c->gscale + 2 * c->n_chunks, parts, T, e, ld, center},
      {V, c->v_codes + off / 2, c->v_scales + off / 16, c->gscale + 2 * c->n_chunks + 1,
       parts + kQuantWs, T, e, ld}};
  nvfp4::ChunkMark mark{c->chunk_start, c->n_chunks + 1, c->n_tokens + T};
  s = launched(nvfp4::launch_quantize(jobs, 2, st, &mark, (qflags & NVFP4_Q_ADAPTIVE_4_6) != 0), st,
               "kv_append");
  if (s) return s;
  c->n_tokens += T;
  c->n_chunks += 1;
  return NVFP4_OK;
}

int nvfp4_kv_append(nvfp4_kv_cache *c, const uint16_t *K, const uint16_t *V, int64_t T, int64_t ld,
                    void *ws, size_t ws_bytes, void *stream) {
  return nvfp4_kv_append_ex(c, K, V, T, ld, 0u, ws, ws_bytes, stream);
}

// nvfp4_qkv_append workspace: [linear workspace | tile maxima]; the append of
// K and V (the unfused fallback) uses regions 0 and 1 of the head, after the
// quantisation of x in region 0 is done
struct QkvWs {
  LinearWs lin;
  size_t slots, total;
  int64_t max_tiles;
};

static QkvWs qkv_ws(int64_t T, int64_t N, int64_t D) {
  QkvWs w;
  w.lin = linear_ws(T, D);
  w.max_tiles = ((T + 127) / 128) * ((N + 127) / 128);   // the finest tiling the GEMM uses
  w.slots = w.lin.total;
  w.total = round_up(w.slots + size_t(w.max_tiles) * sizeof(uint32_t), 256);
  return w;
}

int nvfp4_qkv_append_workspace(int64_t T, int64_t heads, int64_t head_dim, int64_t D, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  int s;
  if ((s = check_mk(T, D, "qkv_append_workspace"))) return s;
  if (heads < 1 || head_dim < 32 || head_dim % 32) return fail(NVFP4_EINVAL, "qkv_append_workspace: bad heads or head_dim");
  const int64_t N = 3 * heads * head_dim;
  if (N > kMaxElements / D || T > kMaxElements / N) return fail(NVFP4_EINVAL, "qkv_append_workspace: problem too large");
  *bytes = qkv_ws(T, N, D).total;
  return NVFP4_OK;
}

int nvfp4_qkv_append(nvfp4_kv_cache *c, const uint16_t *x, int64_t T, int64_t D, const uint8_t *Wq,
                     const uint8_t *Ws, const float *Wg, const uint16_t *bias, uint16_t *QKV,
                     uint32_t qflags, void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_cache(c, "qkv_append"))) return s;
  if (qflags & ~NVFP4_Q_ADAPTIVE_4_6) return fail(NVFP4_EINVAL, "qkv_append: unknown flags");
  size_t need = 0;
  if ((s = nvfp4_qkv_append_workspace(T, c->heads, c->head_dim, D, &need))) return s;
  const int64_t hd = c->heads * c->head_dim, N = 3 * hd;
  if ((s = check_gemm_args(nullptr, nullptr, nullptr, Wq, Ws, Wg, bias, QKV, T, N, D, 0u, false))) return s;
  if ((s = check_ptr(x, "x"))) return s;
  if (T > c->capacity - c->n_tokens) return fail(NVFP4_ECAPACITY, "qkv_append: token capacity exceeded");
  if (c->n_chunks >= c->max_chunks) return fail(NVFP4_ECAPACITY, "qkv_append: no chunk slot left");
  const QkvWs w = qkv_ws(T, N, D);
  if (c->k_center != nullptr) need = smooth_ws(w.total, T, hd).total;
  if (ws == nullptr || ws_bytes < need) return fail(NVFP4_EWORKSPACE, "qkv_append: workspace too small");
  if ((s = check_ptr(ws, "ws"))) return s;
  uint8_t *base = static_cast<uint8_t *>(ws);
  uint8_t *aq = base + w.lin.codes;
  uint8_t *as = base + w.lin.scales;
  float *ag = reinterpret_cast<float *>(base + w.lin.gscale);
  uint32_t *slots = reinterpret_cast<uint32_t *>(base + w.slots);
  hipStream_t st = static_cast<hipStream_t>(stream);
  nvfp4::QuantJob jx{x, aq, as, ag, base + w.lin.partials, T, D, D};
  if ((s = launched(nvfp4::launch_quantize(&jx, 1, st), st, "qkv_append/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, QKV, T, N, D, 0u};
  int bm = 0, bn = 0;
  nvfp4::gemm_tile_of(a, &bm, &bn);
  // fused when every tile's columns lie inside one of Q, K, V (and the keys
  // are quantised as they are: a K-smoothed cache quantises centred keys,
  // whose maximum the GEMM tiles do not see)
  const bool fused = hd % bn == 0 && c->k_center == nullptr;
  if (fused) {
    a.tile_amax = slots;
    if (nvfp4::gemm_tile_count(a) > w.max_tiles) return fail(NVFP4_EHIP, "qkv_append: internal tile count exceeds the workspace");
  }
  if ((s = launched(nvfp4::launch_gemm(a, st), st, "qkv_append/gemm"))) return s;
  const int64_t off = c->n_tokens * hd;
  const uint16_t *center = nullptr;
  if (c->k_center != nullptr &&
      (s = enqueue_smoothing(c, QKV + hd, T, N, base, w.total, st, "qkv_append/smooth", &center)))
    return s;
  nvfp4::QuantJob jobs[2] = {
      {QKV + hd, c->k_codes + off / 2, c->k_scales + off / 16, c->gscale + 2 * c->n_chunks, base, T, hd, N,
       center},
      {QKV + 2 * hd, c->v_codes + off / 2, c->v_scales + off / 16, c->gscale + 2 * c->n_chunks + 1,
       base + kQuantWs, T, hd, N}};
  const nvfp4::ChunkMark mark{c->chunk_start, c->n_chunks + 1, c->n_tokens + T};
  const bool adapt = (qflags & NVFP4_Q_ADAPTIVE_4_6) != 0;
  if (fused) {
    const int64_t tiles_m = (T + bm - 1) / bm, per = (hd / bn) * tiles_m;
    const uint32_t *const maxima[2] = {slots + per, slots + 2 * per};
    s = launched(nvfp4::launch_encode2_from_partials(jobs, maxima, per, mark, adapt, st), st, "qkv_append/encode");
  } else {
    s = launched(nvfp4::launch_quantize(jobs, 2, st, &mark, adapt), st, "qkv_append/append");
  }
  if (s) return s;
  c->n_tokens += T;
  c->n_chunks += 1;
  return NVFP4_OK;
}

int nvfp4_kv_dequant(const nvfp4_kv_cache *c, int64_t t0, int64_t t1, uint16_t *K_out,
                     uint16_t *V_out, void *stream) {
  int s;
  if ((s = check_cache(c, "kv_dequant"))) return s;
  if (t0 < 0 || t1 < t0 || t1 > c->n_tokens) return fail(NVFP4_EINVAL, "kv_dequant: range outside the filled cache");
  if (t0 == t1) return NVFP4_OK;                       // nothing to write, outputs unused
  if ((s = check_ptr(K_out, "K_out"))) return s;
  if ((s = check_ptr(V_out, "V_out"))) return s;
  nvfp4::KvDequantArgs a{};
  a.codes[0] = c->k_codes;
  a.codes[1] = c->v_codes;
  a.scales[0] = c->k_scales;
  a.scales[1] = c->v_scales;
  a.out[0] = K_out;
  a.out[1] = V_out;
  a.gscale = c->gscale;
  a.chunk_start = c->chunk_start;
  a.n_chunks = c->n_chunks;
  a.t0 = t0;
  a.t1 = t1;
  a.elems_per_token = c->heads * c->head_dim;
  a.kcenter = c->k_center;
  return launched(nvfp4::launch_kv_dequant(a, static_cast<hipStream_t>(stream)),
                  static_cast<hipStream_t>(stream), "kv_dequant");
}

// ---------------------------------------------------------------------------
// Attention over the NVFP4 cache and its bf16 twin

static size_t attention_ws_bytes(int64_t Tq, int64_t heads, int64_t Tk) {
  const int64_t ns = nvfp4::attention_splits(Tq, heads, Tk);
  const int64_t kps = nvfp4::attention_keys_per_split(Tk, ns);
  const int64_t nsplit = (Tk + kps - 1) / kps;
  if (nsplit <= 1) return 0;
  const size_t rows = size_t(nsplit) * size_t(Tq) * size_t(heads);
  // the split results after the common head
  return kWsHead + round_up(rows * 128 * sizeof(float), 256) + round_up(rows * 2 * sizeof(float), 256);
}

static int check_attn_common(const uint16_t *Q, int64_t Tq, int64_t ldq, int64_t heads, uint16_t *O,
                             int64_t ldo, float scale, const char *who) {
  int s;
  if (Tq < 1) return fail(NVFP4_EINVAL, std::string(who) + ": Tq must be >= 1");
  if (heads < 1) return fail(NVFP4_EINVAL, std::string(who) + ": heads must be >= 1");
  if (ldq < heads * 128 || ldq % 8 || ldo < heads * 128 || ldo % 8)
    return fail(NVFP4_EINVAL, std::string(who) + ": ldq and ldo must be >= heads*128 and multiples of 8");
  if (Tq > kMaxElements / ldq || Tq > kMaxElements / ldo) return fail(NVFP4_EINVAL, std::string(who) + ": Tq too large");
  if (!(scale >= 0.0f) || scale > 3.0e38f) return fail(NVFP4_EINVAL, std::string(who) + ": scale must be finite and >= 0");
  if ((s = check_ptr(Q, "Q"))) return s;
  if ((s = check_ptr(O, "O"))) return s;
  return NVFP4_OK;
}

static int run_attention(nvfp4::AttnArgs &a, bool bf16, float scale, void *ws, size_t ws_bytes,
                         void *stream, const char *who) {
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(128.0f);
  a.qk_scale = sc * 1.4426950408889634f;
  const int64_t ns = nvfp4::attention_splits(a.Tq, a.heads, a.Tk);
  a.keys_per_split = nvfp4::attention_keys_per_split(a.Tk, ns);
  a.nsplit = (int)((a.Tk + a.keys_per_split - 1) / a.keys_per_split);
  const size_t need = attention_ws_bytes(a.Tq, a.heads, a.Tk);
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (a.nsplit > 1) {
    if (ws == nullptr || ws_bytes < need) return fail(NVFP4_EWORKSPACE, std::string(who) + ": workspace too small");
    int s;
    if ((s = check_ptr(ws, "ws"))) return s;
    const size_t rows = size_t(a.nsplit) * size_t(a.Tq) * size_t(a.heads);
    uint8_t *parts = static_cast<uint8_t *>(ws) + kWsHead;
    a.part_o = reinterpret_cast<float *>(parts);
    a.part_ml = reinterpret_cast<float *>(parts + round_up(rows * 128 * sizeof(float), 256));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(nvfp4::launch_attention(a, bf16, st), st, who);
}

int nvfp4_quantize_rht_workspace(int64_t T, int64_t N, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  if (T < 32 || T % 32) return fail(NVFP4_EINVAL, "quantize_rht_workspace: T must be a positive multiple of 32");
  if (N < 1 || N > kMaxElements / T) return fail(NVFP4_EINVAL, "quantize_rht_workspace: bad N");
  *bytes = kWsHead + 4 * size_t(nvfp4::kRhtMaxParts);     // partial maxima after the common head
  return NVFP4_OK;
}

int nvfp4_quantize_rht(const uint16_t *x, int64_t T, int64_t N, int64_t ldx, uint32_t sign_mask,
                       uint8_t *codes, uint8_t *scales, float *gscale, void *ws, size_t ws_bytes,
                       void *stream) {
  int s;
  size_t need = 0;
  if ((s = nvfp4_quantize_rht_workspace(T, N, &need))) return s;
  if (ldx < N || ldx % 8) return fail(NVFP4_EINVAL, "quantize_rht: ldx must be >= N and a multiple of 8");
  if (ldx > kMaxElements / T) return fail(NVFP4_EINVAL, "quantize_rht: ldx*T too large");
  if (sign_mask >> 16) return fail(NVFP4_EINVAL, "quantize_rht: sign_mask has 16 bits");
  if ((s = check_ptr(x, "x"))) return s;
  if ((s = check_ptr(codes, "codes"))) return s;
  if ((s = check_ptr(scales, "scales"))) return s;
  if ((s = check_ptr(gscale, "gscale", 4))) return s;
  if (ws == nullptr || ws_bytes < need) return fail(NVFP4_EWORKSPACE, "quantize_rht: workspace too small");
  if ((s = check_ptr(ws, "ws", 4))) return s;
  nvfp4::RhtArgs a{x, T, N, ldx, sign_mask, codes, scales, gscale,
                   reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ws) + kWsHead)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launched(nvfp4::launch_quantize_rht(a, st), st, "quantize_rht");
}

int nvfp4_kv_attention_workspace(int64_t Tq, int64_t heads, int64_t Tk, size_t *bytes) {
  if (bytes == nullptr) return fail(NVFP4_EINVAL, "bytes is NULL");
  if (Tq < 1 || heads < 1 || Tk < 1) return fail(NVFP4_EINVAL, "kv_attention_workspace: Tq, heads and Tk must be >= 1");
  if (Tq > kMaxElements / (heads * 128)) return fail(NVFP4_EINVAL, "kv_attention_workspace: Tq too large");
  *bytes = attention_ws_bytes(Tq, heads, Tk);
  return NVFP4_OK;
}

int nvfp4_kv_attention(const nvfp4_kv_cache *c, const uint16_t *Q, int64_t Tq, int64_t ldq,
                       const int64_t *ranges, int n_ranges, float scale, uint16_t *O, int64_t ldo,
                       void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_cache(c, "kv_attention"))) return s;
  if (c->head_dim != 128) return fail(NVFP4_EINVAL, "kv_attention: head_dim must be 128");
  if ((s = check_attn_common(Q, Tq, ldq, c->heads, O, ldo, scale, "kv_attention"))) return s;
  if (ranges == nullptr || n_ranges < 1 || n_ranges > NVFP4_ATTN_MAX_RANGES)
    return fail(NVFP4_EINVAL, "kv_attention: between 1 and NVFP4_ATTN_MAX_RANGES token ranges are required");
  nvfp4::AttnArgs a{};
  int64_t Tk = 0;
  for (int i = 0; i < n_ranges; ++i) {
    const int64_t lo = ranges[2 * i], hi = ranges[2 * i + 1];
    if (lo < 0 || hi <= lo || hi > c->n_tokens)
      return fail(NVFP4_EINVAL, "kv_attention: each range must be a non-empty [start, end) inside the filled cache");
    for (int j = 0; j < i; ++j)
      if (lo < ranges[2 * j + 1] && ranges[2 * j] < hi) return fail(NVFP4_EINVAL, "kv_attention: ranges overlap");
    a.range_lo[i] = lo;
    a.range_len[i] = hi - lo;
    Tk += hi - lo;
  }
  if (c->n_tokens >= (int64_t(1) << 24) || c->n_tokens * c->heads * 128 > (int64_t(1) << 31))
    return fail(NVFP4_EINVAL, "kv_attention: the cache must hold fewer than 2^24 tokens and at most 2^31 elements per tensor");
  a.n_ranges = n_ranges;
  a.Tk = Tk;
  a.kv_tokens = c->n_tokens;
  a.q = Q;
  a.ldq = ldq;
  a.o = O;
  a.ldo = ldo;
  a.Tq = Tq;
  a.heads = c->heads;
  a.kc = c->k_codes;
  a.ks = c->k_scales;
  a.vc = c->v_codes;
  a.vs = c->v_scales;
  a.gscale = c->gscale;
  a.chunk_start = c->chunk_start;
  a.n_chunks = c->n_chunks;
  a.kcenter = c->k_center;
  return run_attention(a, false, scale, ws, ws_bytes, stream, "kv_attention");
}

int nvfp4_attention_bf16(const uint16_t *Q, int64_t Tq, int64_t ldq, const uint16_t *K, const uint16_t *V,
                         int64_t Tk, int64_t ldkv, int64_t heads, float scale, uint16_t *O, int64_t ldo,
                         void *ws, size_t ws_bytes, void *stream) {
  int s;
  if ((s = check_attn_common(Q, Tq, ldq, heads, O, ldo, scale, "attention_bf16"))) return s;
  if (Tk < 1) return fail(NVFP4_EINVAL, "attention_bf16: Tk must be >= 1");
  if (ldkv < heads * 128 || ldkv % 8) return fail(NVFP4_EINVAL, "attention_bf16: ldkv must be >= heads*128 and a multiple of 8");
  if (Tk >= (int64_t(1) << 24) || Tk * ldkv > (int64_t(1) << 30))
    return fail(NVFP4_EINVAL, "attention_bf16: Tk must be below 2^24 and Tk*ldkv at most 2^30 (K and V below 2^31 bytes)");
  if ((s = check_ptr(K, "K"))) return s;
  if ((s = check_ptr(V, "V"))) return s;
  nvfp4::AttnArgs a{};
  a.range_lo[0] = 0;
  a.range_len[0] = Tk;
  a.n_ranges = 1;
  a.Tk = Tk;
  a.kv_tokens = Tk;
  a.q = Q;
  a.ldq = ldq;
  a.o = O;
  a.ldo = ldo;
  a.Tq = Tq;
  a.heads = heads;
  a.kb = K;
  a.vb = V;
  a.ldkv = ldkv;
  return run_attention(a, true, scale, ws, ws_bytes, stream, "attention_bf16");
}

uint64_t nvfp4_testing_set_quantize_wait(uint64_t ticks) { return nvfp4::set_resident_wait_ticks(ticks); }

int nvfp4_testing_set_launch_events(void *const *events, int count) {
  if (count < 0 || (count > 0 && events == nullptr))
    return fail(NVFP4_EINVAL, "testing_set_launch_events: bad event list");
  g_events_left.store(0, std::memory_order_relaxed);
  g_events.store(events, std::memory_order_relaxed);
  g_events_next.store(0, std::memory_order_relaxed);
  g_events_left.store(count, std::memory_order_relaxed);
  return NVFP4_OK;
}

const char *nvfp4_strerror(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_EINVAL: return "invalid argument";
    case NVFP4_EWORKSPACE: return "workspace too small";
    case NVFP4_ECAPACITY: return "KV cache capacity exceeded";
    case NVFP4_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *nvfp4_last_error(void) { return g_last_error; }

}  // extern "C"
