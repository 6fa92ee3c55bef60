// C ABI of the NVFP4 library: argument validation, workspace layout and
// kernel launches.  Every entry point is declared (with its contract) in
// include/nvfp4.h.
#include <nvfp4.h>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string &msg) {
  g_last_error = msg;
  return status;
}

bool aligned(const void *p, size_t a = NVFP4_ALIGN) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxElements = int64_t(1) << 36;   // keeps unit indices below 2^31
constexpr size_t kQuantWs = nvfp4::kQuantScratchBytes;

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

// nvfp4_linear workspace: [codes | scales | gscale | amax partials]
struct LinearWs {
  size_t codes, scales, gscale, partials, total;
};

LinearWs linear_ws(int64_t M, int64_t K) {
  LinearWs w;
  const size_t n = size_t(M) * size_t(K);
  w.codes = 0;
  w.scales = round_up(w.codes + n / 2, 256);
  w.gscale = round_up(w.scales + n / 16, 256);
  w.partials = round_up(w.gscale + sizeof(float), 256);
  w.total = round_up(w.partials + kQuantWs, 256);
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
  nvfp4::QuantJob j{x, codes, scales, gscale, static_cast<uint32_t *>(ws), M, K, K};
  return hip_status(nvfp4::launch_quantize(&j, 1, static_cast<hipStream_t>(stream), nullptr,
                                           (qflags & NVFP4_Q_ADAPTIVE_4_6) != 0,
                                           (qflags & NVFP4_Q_BLOCK_2D) != 0),
                    "quantize");
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
  return hip_status(nvfp4::launch_gemm(a, static_cast<hipStream_t>(stream)), "gemm");
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
  nvfp4::QuantJob j{x, aq, as, ag, reinterpret_cast<uint32_t *>(base + w.partials), M, K, K};
  if ((s = hip_status(nvfp4::launch_quantize(&j, 1, st), "linear/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, C, M, N, K, flags};
  return hip_status(nvfp4::launch_gemm(a, st), "linear/gemm");
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
  nvfp4::QuantJob jx{x, aq, as, ag, reinterpret_cast<uint32_t *>(base + w.lin.partials), M, K, K};
  if ((s = hip_status(nvfp4::launch_quantize(&jx, 1, st), "linear_q/quantize"))) return s;
  nvfp4::GemmArgs a{aq, as, ag, Wq, Ws, Wg, bias, H, M, N, K, flags};
  a.tile_amax = slots;
  const int64_t tiles = nvfp4::gemm_tile_count(a);
  if (tiles > w.max_tiles) return fail(NVFP4_EHIP, "linear_q: internal tile count exceeds the workspace");
  if ((s = hip_status(nvfp4::launch_gemm(a, st), "linear_q/gemm"))) return s;
  nvfp4::QuantJob jh{H, Hq, Hs, Hg, slots, M, N, N};
  return hip_status(nvfp4::launch_encode_from_partials(jh, tiles, st), "linear_q/encode");
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
  if (ws == nullptr || ws_bytes < 2 * kQuantWs) return fail(NVFP4_EWORKSPACE, "kv_append: workspace too small");
  if ((s = check_ptr(ws, "ws"))) return s;
  const int64_t e = c->heads * c->head_dim;           // elements per token
  const int64_t off = c->n_tokens * e;
  uint32_t *parts = static_cast<uint32_t *>(ws);
  nvfp4::QuantJob jobs[2] = {
      {K, c->k_codes + off / 2, c->k_scales + off / 16, c->gscale + 2 * c->n_chunks, parts, T, e, ld},
      {V, c->v_codes + off / 2, c->v_scales + off / 16, c->gscale + 2 * c->n_chunks + 1,
       parts + kQuantWs / sizeof(uint32_t), T, e, ld}};
  nvfp4::ChunkMark mark{c->chunk_start, c->n_chunks + 1, c->n_tokens + T};
  s = hip_status(nvfp4::launch_quantize(jobs, 2, static_cast<hipStream_t>(stream), &mark,
                                        (qflags & NVFP4_Q_ADAPTIVE_4_6) != 0),
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
  return hip_status(nvfp4::launch_kv_dequant(a, static_cast<hipStream_t>(stream)), "kv_dequant");
}

uint64_t nvfp4_testing_set_quantize_wait(uint64_t ticks) { return nvfp4::set_resident_wait_ticks(ticks); }

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

const char *nvfp4_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
