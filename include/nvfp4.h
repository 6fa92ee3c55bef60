/*
 * nvfp4.h — C ABI of the MI355X (gfx950) NVFP4 W4A4 linear layer and NVFP4
 * KV cache.
 *
 * Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io
 * reading notes), section 二、方法:
 *   - NVFP4 量化格式: a tensor is stored as E2M1 4-bit elements, one FP8 E4M3
 *     scale per 16 contiguous elements and one FP32 scale per tensor;
 *     Dequant(X) = X^FP4 · α^FP8 · α^FP32.
 *   - NVFP4 训练的工程细节: weights and activations are both 4-bit (W4A4);
 *     activations use 1-D block scaling; reductions stay in higher precision.
 *   - 推理底座: weights are materialised once in 4 bits; the KV cache is
 *     quantised again per chunk (4·T·H·d → 9/8·T·H·d bytes) and read back
 *     through a dequantisation kernel.
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  bf16 values travel as uint16_t
 *     bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work; none synchronises the host.  Results (including
 *     the FP32 tensor scale) stay in device memory.
 *   - Return value: NVFP4_OK (0) or a positive status code.  Argument errors are
 *     detected on the host before anything is enqueued and leave every output
 *     untouched.  A kernel fault surfaces at the caller's next synchronisation.
 *     No C++ exception crosses this interface.  nvfp4_last_error() gives a
 *     message for the calling thread's last failure.
 *   - Preconditions not checked on the device: bf16 inputs are finite and a
 *     tensor's largest magnitude is 0 or at least 2^-100.
 *   - Layouts are row-major and dense.  A row of K elements occupies K/2 code
 *     bytes (element 2j in the low nibble of byte j) and K/16 scale bytes
 *     (E4M3, block b covers elements 16b..16b+15).
 *   - Concurrency: calls are reentrant; calls that share an output buffer or a
 *     KV cache must be ordered by the caller (same stream, or events).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define NVFP4_OK          0
#define NVFP4_EINVAL      1  /* null pointer, bad size, misalignment, unknown flag */
#define NVFP4_EWORKSPACE  2  /* workspace missing or smaller than required       */
#define NVFP4_ECAPACITY   3  /* KV cache token capacity or chunk slots exhausted */
#define NVFP4_EHIP        4  /* the HIP runtime reported an error at launch      */

/* flags for nvfp4_gemm / nvfp4_linear */
#define NVFP4_EPI_GELU_TANH 0x1u  /* apply tanh-form GELU before the bf16 cast */
/* Optional workgroup-tile choice (a performance hint; 0 = automatic).  The
 * result does not depend on it beyond fp32 summation order. */
#define NVFP4_TILE_MASK     0xF00u
#define NVFP4_TILE_256x256  0x100u
#define NVFP4_TILE_256x192  0x200u
#define NVFP4_TILE_192x256  0x300u
#define NVFP4_TILE_256x128  0x400u
#define NVFP4_TILE_128x256  0x500u
#define NVFP4_TILE_128x128  0x600u

/* flags for nvfp4_quantize_ex / nvfp4_kv_append_ex */
/* Adaptive {4, 6} block scales: each 16-block is encoded with its amax mapped
 * to 6 and to 4 and the encoding with the smaller binary32 squared error is
 * kept (ties to 6).  The output format is unchanged. */
#define NVFP4_Q_ADAPTIVE_4_6 0x10u
/* Two-dimensional 16x16 blocks for weights (nvfp4_quantize_ex only): one
 * scale per tile of 16 rows x 16 elements, stored on each of its rows. */
#define NVFP4_Q_BLOCK_2D 0x20u

/* Alignment every device pointer must satisfy (bytes). */
#define NVFP4_ALIGN 16

/*
 * Workspace bytes nvfp4_quantize needs for an [M, K] input (scratch for the
 * tensor-amax reduction).  Writes *bytes; the size depends only on M and K.
 *
 * Workspaces of every call (quantise, linear, linear_q, KV append, QKV
 * append, Hadamard-transformed quantise, attention) must be all zero before
 * their first use (hipMemset, or a zero-filled tensor); after that only the
 * library writes them, and the caller must not change them between calls.
 * The library keeps a call counter in them from one call to the next, in
 * device memory, so calls captured in a HIP graph stay correct on every
 * replay.  Every workspace starts with the same 24 KiB head, the scratch of
 * two quantised tensors, which only the quantiser writes; each call's other
 * buffers lie after it.  So one buffer, sized for the largest of its uses,
 * may be shared by calls of any kind and size that are ordered on one
 * stream; calls that may run at the same time need separate workspaces.
 */
int nvfp4_quantize_workspace(int64_t M, int64_t K, size_t *bytes);

/*
 * Dynamic NVFP4 quantisation of a bf16 matrix (the per-call activation
 * quantiser of W4A4 inference; also the offline weight quantiser).
 * Source: 二、方法 / NVFP4 量化格式 (three-level scaling) and
 * NVFP4 训练的工程细节 (1-D block scaling of activations).
 *
 *   x       bf16 [M, K] row-major, 16-byte aligned
 *   codes   out: uint8 [M, K/2]   E2M1 codes, two per byte
 *   scales  out: uint8 [M, K/16]  E4M3 block scales
 *   gscale  out: float [1]        FP32 tensor scale g
 *   ws      scratch of at least nvfp4_quantize_workspace(M, K) bytes
 *
 * Arithmetic (binary32, nearest-even, subnormals kept): A = max|x|;
 * g = A/2688 (g = 1 when A = 0); per 16-block S = E4M3_rne_satfinite(a/(6g));
 * r = 1/(S·g) (0 when S = 0); code = sign(x)·8 | E2M1_rne_sat(|x|·r).
 * Requires M >= 1, K >= 32, K % 32 == 0.
 */
int nvfp4_quantize(const uint16_t *x, int64_t M, int64_t K,
                   uint8_t *codes, uint8_t *scales, float *gscale,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_quantize with quantiser flags (0, NVFP4_Q_ADAPTIVE_4_6 or
 * NVFP4_Q_BLOCK_2D; the two flags exclude each other).
 * Source of the adaptive mode: 二、方法 / 推理底座 (adaptive scale selection for
 * the KV chunks) and the distillation paragraph of 二、方法 (amax targets
 * {4, 6}).  With the flag, each 16-block is encoded twice: as above, and with
 * the divisor 4g in place of 6g (S4 = E4M3_rne_satfinite(a/(4g)),
 * r4 = 1/(S4·g)).  For each encoding err = Σ_i fl(e_i·e_i) accumulated in
 * binary32 in element order, e_i = fl(x_i − fl(fl(E2M1_i·S)·g)) with the
 * code's sign; the amax→4 encoding is kept only when its err is smaller.
 * NVFP4_Q_BLOCK_2D, for weights (二、方法 / NVFP4 训练的工程细节: blocks along
 * two dimensions, so W and its transpose share one quantisation): a block is
 * 16 consecutive rows (groups from row 0; the last may be shorter) by 16
 * elements along K; a = the tile's max |x|, S and r as above, and the scale
 * byte is stored on every row of the tile, so the scales keep the
 * [M, K/16] layout and nvfp4_gemm takes such weights unchanged.  Two launches.
 * Returns NVFP4_EINVAL for unknown or combined flags; other arguments as
 * nvfp4_quantize.
 */
int nvfp4_quantize_ex(const uint16_t *x, int64_t M, int64_t K, uint32_t qflags,
                      uint8_t *codes, uint8_t *scales, float *gscale,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * W4A4 GEMM with FP32 accumulation and a bf16 epilogue:
 *   C[m, n] = bf16( fl32( fl32(acc[m, n] · fl32(Ag·Wg)) + bias[n] ) [→ GELU] )
 *   acc[m, n] = Σ_k (E2M1(Aq[m,k])·E4M3(As[m,k/16])) · (E2M1(Wq[n,k])·E4M3(Ws[n,k/16]))
 * Source: 二、方法 / NVFP4 量化格式 (Dequant = X^FP4·α^FP8·α^FP32) and
 * 推理底座 (W4A4 inference with weights materialised once in 4 bits).
 *
 *   Aq, As, Ag  activations: codes [M, K/2], scales [M, K/16], tensor scale [1]
 *   Wq, Ws, Wg  weights (one output channel per row): codes [N, K/2],
 *               scales [N, K/16], tensor scale [1]
 *   bias        bf16 [N] or NULL
 *   C           out: bf16 [M, N] row-major
 *   flags       NVFP4_EPI_GELU_TANH and/or one NVFP4_TILE_* hint (or 0)
 * GELU is the tanh form 0.5·y·(1 + tanh(√(2/π)·(y + 0.044715·y³))), evaluated
 * in binary32 as y·rcp(1 + 2^(y·(c1 + c2·y²))), c1 = −2·log2(e)·√(2/π),
 * c2 = 0.044715·c1 (relative error below 1e-5 before the bf16 cast).
 * Requires M, N >= 1, K >= 32, K % 32 == 0.  Every scale byte must be a
 * finite E4M3 value (not 0x7F/0xFF).
 */
int nvfp4_gemm(const uint8_t *Aq, const uint8_t *As, const float *Ag,
               const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
               const uint16_t *bias, uint16_t *C,
               int64_t M, int64_t N, int64_t K, uint32_t flags, void *stream);

/* Workspace bytes nvfp4_linear_q needs (includes the bf16 [M, N] output). */
int nvfp4_linear_q_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes);

/*
 * A linear layer whose bf16 output H is handed on in NVFP4, as the input of
 * the next W4A4 layer (the FFN up projection feeding the down projection):
 *   H = nvfp4_linear(x, W, bias, flags);  (Hq, Hs, Hg) = nvfp4_quantize(H)
 * with exactly those bytes.  Source: 二、方法 / 推理底座 (W4A4 inference) and
 * 二、方法 / NVFP4 量化格式.  The GEMM epilogue records each output tile's
 * largest |H|, so H (kept in the workspace) is read once by the encoder
 * instead of twice.
 *   x, Wq, Ws, Wg, bias, M, N, K, flags   as for nvfp4_linear (C is internal)
 *   Hq  out: uint8 [M, N/2];  Hs  out: uint8 [M, N/16];  Hg  out: float [1]
 *   ws  scratch of at least nvfp4_linear_q_workspace(M, N, K) bytes; the
 *       bf16 H sits inside it and is overwritten by the next call.
 * Requires N % 32 == 0 besides nvfp4_linear's conditions.
 */
int nvfp4_linear_q(const uint16_t *x, const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                   const uint16_t *bias, int64_t M, int64_t N, int64_t K, uint32_t flags,
                   uint8_t *Hq, uint8_t *Hs, float *Hg, void *ws, size_t ws_bytes, void *stream);

/*
 * Largest activation (M·K elements) nvfp4_linear_noalloc accepts: its built-in
 * workspace holds the NVFP4 activation of that size (36 MiB per device).
 */
#define NVFP4_NOALLOC_MAX_ELEMENTS (1LL << 26)

/*
 * nvfp4_linear without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, arithmetic and bytes as
 * nvfp4_linear; the quantised activation and the quantiser's scratch live in
 * an array of the library's own device memory (one per device, zero at load,
 * held until the process ends).  Calls nothing that allocates.
 *   Requires M·K <= NVFP4_NOALLOC_MAX_ELEMENTS (else NVFP4_EINVAL, with the
 *   limit in the message), besides nvfp4_linear's conditions.
 *   Every call on one device shares that device's array: calls that may
 *   overlap on one device (different streams without ordering) race and give
 *   undefined results.  Calls ordered on one stream are safe in any sequence
 *   of sizes.
 */
int nvfp4_linear_noalloc(const uint16_t *x,
                         const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                         const uint16_t *bias, uint16_t *C,
                         int64_t M, int64_t N, int64_t K, uint32_t flags, void *stream);

/*
 * Workgroup tile (rows of A x rows of W) nvfp4_gemm uses for an M x N x K
 * problem; informational (for reporting), enqueues nothing.
 */
int nvfp4_gemm_tile(int64_t M, int64_t N, int64_t K, int *bm, int *bn);

/* Workspace bytes nvfp4_linear needs for an [M, K] activation. */
int nvfp4_linear_workspace(int64_t M, int64_t K, size_t *bytes);

/*
 * The W4A4 linear layer: nvfp4_quantize(x) into the workspace, then
 * nvfp4_gemm against pre-quantised weights, on one stream.
 *   x   bf16 [M, K];  other arguments as for nvfp4_gemm;
 *   ws  scratch of at least nvfp4_linear_workspace(M, K) bytes.
 */
int nvfp4_linear(const uint16_t *x,
                 const uint8_t *Wq, const uint8_t *Ws, const float *Wg,
                 const uint16_t *bias, uint16_t *C,
                 int64_t M, int64_t N, int64_t K, uint32_t flags,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * NVFP4 KV cache.  Source: 二、方法 / 推理底座 (the KV cache is quantised per
 * chunk in place and read back through a dequantisation kernel; storage
 * 9/8·T·H·d bytes for K and V together).
 *
 * The caller allocates the device buffers and fills the geometry and pointer
 * fields; nvfp4_kv_init validates them and zeroes the counters.  The counters
 * are host-side state maintained by the library; do not edit them.  Each
 * append quantises K and V (each viewed as [T·H, head_dim], blocks of 16
 * along head_dim) with its own pair of tensor scales and writes them at token
 * offset n_tokens.
 *
 * K-smoothing (二、方法 / 推理底座 names it for the keys of each KV chunk and
 * does not define it; the definition used): when k_center is not NULL, every
 * append first takes the centre of each key channel over its T tokens,
 *     μ = bf16_rne( fl64( fl64(Σ_t clamp(rne(K·2^24), ±2^38)) / T ) · 2^-24 )
 * (an exact integer sum on a 2^-24 grid, so the result does not depend on
 * summation order), stores it as row n_chunks of k_center, and quantises the
 * smoothed keys bf16_rne(fl32(K − μ)) in place of K.  Read-back and attention
 * add μ back (see nvfp4_kv_dequant, nvfp4_kv_attention).  V is not smoothed.
 * The choice is made once, at nvfp4_kv_init, for every append of the cache.
 */
typedef struct nvfp4_kv_cache {
    int64_t capacity;      /* tokens the buffers hold                        */
    int64_t heads;         /* H                                              */
    int64_t head_dim;      /* d, multiple of 32                              */
    int64_t max_chunks;    /* appends the gscale / chunk_start arrays hold   */
    uint8_t *k_codes;      /* device [capacity, heads, head_dim/2]           */
    uint8_t *k_scales;     /* device [capacity, heads, head_dim/16]          */
    uint8_t *v_codes;      /* device [capacity, heads, head_dim/2]           */
    uint8_t *v_scales;     /* device [capacity, heads, head_dim/16]          */
    float *gscale;         /* device [max_chunks, 2]: (g_K, g_V) per append  */
    int64_t *chunk_start;  /* device [max_chunks + 1]: first token per chunk */
    int64_t n_tokens;      /* host counter: tokens written                   */
    int64_t n_chunks;      /* host counter: appends made                     */
    uint16_t *k_center;    /* device [max_chunks, heads, head_dim] bf16 key
                              centres (16-byte aligned), or NULL: no
                              K-smoothing.  Requires heads·head_dim <= 2^20. */
} nvfp4_kv_cache;

/* Validate geometry and pointers, zero the counters.  Enqueues nothing. */
int nvfp4_kv_init(nvfp4_kv_cache *c);

/* Workspace bytes nvfp4_kv_append needs for an append of T tokens. */
int nvfp4_kv_append_workspace(int64_t T, int64_t heads, int64_t head_dim, size_t *bytes);

/* Extra workspace bytes an append of T tokens to a K-smoothed cache needs,
 * placed after the workspace of nvfp4_kv_append (or nvfp4_qkv_append): the
 * channel sums of each strip of tokens.  This part needs no
 * initialisation. */
int nvfp4_kv_smooth_workspace(int64_t T, int64_t heads, int64_t head_dim, size_t *bytes);

/*
 * Quantise K and V (bf16, T tokens of [heads, head_dim]) into the cache at
 * token offset c->n_tokens, record their tensor scales as chunk c->n_chunks,
 * then advance the counters.  Returns NVFP4_ECAPACITY (cache unchanged) when
 * the tokens or the chunk slots would overflow.  T >= 1.
 *   ld  elements from one token's first element to the next token's, in both
 *       K and V: heads·head_dim for dense [T, heads, head_dim] tensors, or the
 *       row length of a fused QKV projection output whose K and V column
 *       slices are passed directly.  ld >= heads·head_dim, ld % 8 == 0.
 */
int nvfp4_kv_append(nvfp4_kv_cache *c, const uint16_t *K, const uint16_t *V, int64_t T,
                    int64_t ld, void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_kv_append with quantiser flags (0 or NVFP4_Q_ADAPTIVE_4_6, as for
 * nvfp4_quantize_ex; 二、方法 / 推理底座 selects adaptive scales for the KV
 * chunks).  The flag may differ between appends: dequantisation reads every
 * chunk the same way.  Returns NVFP4_EINVAL for unknown flags.
 */
int nvfp4_kv_append_ex(nvfp4_kv_cache *c, const uint16_t *K, const uint16_t *V, int64_t T,
                       int64_t ld, uint32_t qflags, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes nvfp4_qkv_append needs (zero before its first use, as for
 * nvfp4_linear; the library keeps it valid from one call to the next). */
int nvfp4_qkv_append_workspace(int64_t T, int64_t heads, int64_t head_dim, int64_t D, size_t *bytes);

/*
 * The QKV projection of T tokens with its K and V appended to the cache, in
 * three launches: quantise x, the W4A4 GEMM, and one encode of the K and V
 * column slices of its output into the cache.  Source: 二、方法 / 推理底座 (W4A4
 * inference; the KV cache is quantised to NVFP4 per chunk as it is written).
 * The result equals nvfp4_linear followed by nvfp4_kv_append_ex on the K and
 * V slices of its output (ld = 3·heads·head_dim), byte for byte, but the
 * append's tensor amax comes from the GEMM epilogue (the largest stored
 * |output| of each workgroup tile), so no pass over K and V precedes the
 * encode.  If the GEMM's tile width does not divide heads·head_dim, the
 * append runs as nvfp4_kv_append_ex does (same bytes, one more pass).
 *   x      bf16 [T, D] activations, 16-byte aligned, D % 32 == 0
 *   Wq/Ws/Wg  NVFP4 weights [3·heads·head_dim, D]: the Q rows, then K, then V
 *   bias   bf16 [3·heads·head_dim] or NULL
 *   QKV    out: bf16 [T, 3·heads·head_dim] (Q for the attention, ldq = 3·heads·head_dim)
 *   qflags 0 or NVFP4_Q_ADAPTIVE_4_6 for the appended K and V
 *   ws     nvfp4_qkv_append_workspace(T, heads, head_dim, D) bytes
 * Errors as nvfp4_linear and nvfp4_kv_append_ex (cache unchanged on error).
 */
int nvfp4_qkv_append(nvfp4_kv_cache *c, const uint16_t *x, int64_t T, int64_t D, const uint8_t *Wq,
                     const uint8_t *Ws, const float *Wg, const uint16_t *bias, uint16_t *QKV,
                     uint32_t qflags, void *ws, size_t ws_bytes, void *stream);

/*
 * Dequantise tokens [t0, t1) of K and V to bf16 [t1-t0, heads, head_dim]:
 *   out = bf16( fl32( fl32(E2M1 · E4M3) · g_chunk ) )
 * (the first product is exact; g_chunk is the tensor scale of the append that
 * wrote the token); keys of a K-smoothed cache are
 *   bf16( fl32( fl32( fl32(E2M1 · E4M3) · g_chunk ) + μ_chunk ) ).
 * Requires 0 <= t0 <= t1 <= c->n_tokens; t0 == t1 is a no-op (the output
 * pointers are then not used and may be NULL).
 */
int nvfp4_kv_dequant(const nvfp4_kv_cache *c, int64_t t0, int64_t t1,
                     uint16_t *K_out, uint16_t *V_out, void *stream);

/*
 * Attention of a chunk of queries over the NVFP4 KV cache, with the cache's
 * dequantisation fused into the kernel.  Source: 二、方法 / 推理底座 (the KV
 * cache is kept in NVFP4 and dequantised by a hand-written kernel inside
 * inference) and 二、方法 / 多镜头注意力锚点 (the KV set of a chunk is the
 * global-sink frames, the shot-sink frames and a window of recent frames,
 * without duplicates).  For each head h and query i:
 *   O[i, h] = softmax_j( Q[i, h] · K[j, h] · scale ) · V[j, h]
 * over the tokens j of `ranges`, with K and V the exact dequantised values
 * E2M1 · E4M3 · g of each token's append (keys of a K-smoothed cache:
 * E2M1 · E4M3 · g + μ, the append's centre; each score then gains Q·μ,
 * computed in fp32 from the fp16 query, once per query and append).
 *   c        cache with head_dim 128 (others: NVFP4_EINVAL)
 *   Q        bf16: query i, head h at Q + i·ldq + 128·h (ldq >= heads·128,
 *            ldq % 8 == 0; Q may be the query slice of a fused QKV output)
 *   ranges   host array of n_ranges (1..NVFP4_ATTN_MAX_RANGES) pairs
 *            [start, end) of disjoint, non-empty token ranges inside the
 *            filled cache; their tokens form the keys, in order
 *   scale    softmax scale; 0 means 1/sqrt(128)
 *   O        out, bf16, same layout as Q with ldo
 *   ws       scratch of nvfp4_kv_attention_workspace(Tq, heads, Tk) bytes
 *            (Tk = total tokens of the ranges; may be 0 bytes, then ws may be
 *            NULL); it needs no initialisation
 * Arithmetic: Q converted to fp16 (exact for |q| in [2^-14, 65504] or 0),
 * K·Q products exact and summed in fp32, times g_K·scale, base-2 online
 * softmax in fp32, P·g_V rounded to bf16, products with V (exact) summed in
 * fp32, one bf16 rounding of the output.  Requires |q| < 65504, and a cache
 * of fewer than 2^24 filled tokens with at most 2^31 elements per tensor
 * (NVFP4_EINVAL otherwise).
 */
#define NVFP4_ATTN_MAX_RANGES 4
int nvfp4_kv_attention_workspace(int64_t Tq, int64_t heads, int64_t Tk, size_t *bytes);
int nvfp4_kv_attention(const nvfp4_kv_cache *c, const uint16_t *Q, int64_t Tq, int64_t ldq,
                       const int64_t *ranges, int n_ranges, float scale,
                       uint16_t *O, int64_t ldo, void *ws, size_t ws_bytes, void *stream);

/*
 * The same attention with bf16 K and V tensors instead of the NVFP4 cache
 * (token j, head h at K + j·ldkv + 128·h): the baseline against which the
 * fused dequantisation's cost is measured.  Q·K and P·V on the bf16 matrix
 * cores (P rounded to bf16), otherwise as nvfp4_kv_attention; the workspace
 * size is nvfp4_kv_attention_workspace(Tq, heads, Tk).  Requires Tk < 2^24
 * and Tk·ldkv <= 2^30 (K and V each below 2^31 bytes).
 */
int nvfp4_attention_bf16(const uint16_t *Q, int64_t Tq, int64_t ldq, const uint16_t *K,
                         const uint16_t *V, int64_t Tk, int64_t ldkv, int64_t heads, float scale,
                         uint16_t *O, int64_t ldo, void *ws, size_t ws_bytes, void *stream);

/*
 * Bytes of scratch nvfp4_quantize_rht needs (8192: one partial maximum per
 * workgroup, written before it is read, so the scratch needs no
 * initialisation).  Fails like nvfp4_quantize_rht on a bad shape.
 */
int nvfp4_quantize_rht_workspace(int64_t T, int64_t N, size_t *bytes);

/*
 * Weight-gradient operand with a random Hadamard transform: transforms x along
 * its token axis and NVFP4-quantises the transpose, so two such operands feed
 * nvfp4_gemm for dW = dyᵀ·x (M = features of dy, N = features of x, K = T).
 * Source: 二、方法 / NVFP4 训练的工程细节 (a random Hadamard transform precedes
 * the quantisation of the weight-gradient GEMM's operands; gradients take 1-D
 * block scales) and 二、方法 / NVFP4 量化格式.
 *
 *   x          bf16 [T, N], token t at x + t·ldx; 16-byte aligned, ldx >= N,
 *              ldx % 8 == 0 (rows 16-byte aligned)
 *   sign_mask  the 16 random signs s_k (bit k set: s_k = −1), drawn by the
 *              caller; pass the same mask for both operands of one product
 *   codes      out: uint8 [N, T/2]  E2M1 codes of the transpose, two per byte,
 *              16-byte aligned (so are scales)
 *   scales     out: uint8 [N, T/16] E4M3 block scales (16 tokens per block)
 *   gscale     out: float [1]       FP32 tensor scale g
 *   ws         scratch of nvfp4_quantize_rht_workspace(T, N) bytes
 *
 * Arithmetic: per group of 16 consecutive tokens (from token 0) and feature n,
 * y = H16·diag(s)·x/4 with Sylvester's H16 (H[i,k] = (−1)^popcount(i&k));
 * the sums are formed exactly (binary64; exact while a group spans less than
 * 2^41 in magnitude) and rounded once to binary32, an exact zero as +0; then
 * the steps of nvfp4_quantize on yᵀ (A = max|y|, g = A/2688, …).  Requires
 * T >= 32, T % 32 == 0 (append zero tokens otherwise: they add nothing to the
 * weight gradient), N >= 1, |x| small enough that y stays finite (below 2^124).
 * Two launches on `stream`.
 */
int nvfp4_quantize_rht(const uint16_t *x, int64_t T, int64_t N, int64_t ldx, uint32_t sign_mask,
                       uint8_t *codes, uint8_t *scales, float *gscale,
                       void *ws, size_t ws_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *nvfp4_strerror(int status);

/* Message for the calling thread's most recent failed call ("" if none). */
const char *nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
