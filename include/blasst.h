/*
 * blasst.h - C ABI of libblasst: BLASST skip-softmax attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (sources: the BLASST explainer post "BLASST: Dynamic BLocked
 * Attention Sparsity via Softmax Thresholding" on the seeallochnaya Telegram
 * channel, and the digg.com thread "BLASST wins Best Paper at MLSys 2026"):
 *
 *   Blocked attention with an online softmax. Keys are cut into tiles of bc
 *   positions and visited in increasing order (post, paragraph "В чём идея").
 *   A running per-row maximum of the scaled scores s = scale * q.k is kept and
 *   earlier partial sums are rescaled when it grows (post, paragraph on the
 *   online trick of FlashAttention 1). A key tile whose maximum falls far below
 *   the running maximum is dropped whole: no exp, no row-sum, no P.V, and its
 *   V rows are never read (post, paragraph beginning "BLASST предлагает"). The
 *   first tile is always processed (post, first figure). The drop test is one
 *   scalar threshold on the online softmax statistics (digg thread).
 *
 *   Precisely, for a query tile (prefill: br rows; decode: one row) and key
 *   tile j (visited left to right):
 *     gap_r = rowmax_r(tile j) - m_r          (m_r = running max; +inf while
 *                                              m_r is -inf; -inf for a row with
 *                                              no visible key in the tile)
 *     g     = max over the tile's valid rows of gap_r
 *     drop  <=>  j > 0  and  g < ln(lambda)    (strict; ln 0 = -inf)
 *   Kept tiles get the usual rescale-and-accumulate. For lambda <= 1 a dropped
 *   tile can never raise the running max, so m_r on entry to tile j equals the
 *   plain prefix max of the row maxima of tiles 0..j-1.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *     allocates no memory and keeps no per-call state; calls are reentrant as
 *     long as concurrent calls do not share a decode workspace.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the legacy
 *     default stream). Outputs are valid once the stream has synchronised.
 *   - All arguments are validated before any HIP call. On any error nothing is
 *     launched and every output is left untouched. No C++ exception crosses
 *     the ABI. Launch failures return BLASST_E_HIP; blasst_last_error() then
 *     holds the HIP error text (thread-local).
 *   - GQA: query head h reads key/value head h / (heads_q / heads_kv).
 *   - Causal prefill is bottom-right aligned: query i sits at key position
 *     len_kv - len_q + i and sees keys 0..len_kv-len_q+i.
 *   - Tensor pointers must be 16-byte aligned, the last dimension must be
 *     contiguous, and every stride times the element size must be a multiple
 *     of 16 bytes (BLASST_E_ALIGN).
 *   - A tensor pointer may be NULL exactly when its tensor has no elements
 *     (batch = 0, or len_q = 0 for the query-side tensors); otherwise a NULL
 *     required pointer is BLASST_E_NULL. A call with no query rows launches
 *     only what fills its non-empty outputs: statistics are zeroed, and the
 *     backward writes zero dk and dv.
 *   - lambda must satisfy 0 <= lambda <= 1 (BLASST_E_LAMBDA otherwise; NaN is
 *     rejected). lambda = 0 drops nothing and gives exact softmax attention.
 *   - scale <= 0 selects 1/sqrt(d_qk); a non-finite scale is BLASST_E_ARG.
 */
#ifndef BLASST_H
#define BLASST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLASST_VERSION 230 /* 2.3.0: two-pass prefill, MXFP4 quantization */

typedef enum blasst_status {
  BLASST_OK = 0,
  BLASST_E_NULL = 1,        /* a required pointer is NULL */
  BLASST_E_SHAPE = 2,       /* bad sizes: negative, heads_q % heads_kv != 0,
                               causal with len_q > len_kv, len_q != 1 for decode */
  BLASST_E_DTYPE = 3,       /* unknown dtype or unsupported input/output pair */
  BLASST_E_LAMBDA = 4,      /* lambda NaN or outside [0, 1] */
  BLASST_E_ALIGN = 5,       /* pointer or stride not 16-byte aligned */
  BLASST_E_UNSUPPORTED = 6, /* valid request with no kernel in this build */
  BLASST_E_ARG = 7,         /* other bad scalar argument (non-finite scale) */
  BLASST_E_HIP = 8,         /* a HIP runtime call failed */
  BLASST_E_WORKSPACE = 9    /* workspace NULL, smaller than the size its
                               query function returns, or not 256-byte
                               aligned */
} blasst_status_t;

typedef enum blasst_dtype {
  BLASST_FP32 = 0, /* float32 */
  BLASST_BF16 = 1  /* bfloat16 */
} blasst_dtype_t;

/* Input and output element types. `dtype` is the type of q, k and v;
 * `out_dtype` the type of out. bfloat16 inputs accumulate in fp32 and may
 * write bfloat16 (rounded to nearest even) or float32 outputs; float32 inputs
 * write float32 outputs. Anything else is BLASST_E_DTYPE. */

/* Sizes and element strides. Strides are in ELEMENTS for the (batch, head,
 * position) dimensions; the last (feature) dimension is contiguous. For
 * decode the query has no position dimension and q_stride[2] / o_stride[2]
 * are ignored. */
typedef struct blasst_shape {
  int32_t batch;    /* B  >= 0 */
  int32_t heads_q;  /* Hq >= 1 */
  int32_t heads_kv; /* Hkv >= 1, divides Hq */
  int32_t len_q;    /* Nq >= 0 (decode: 1) */
  int32_t len_kv;   /* Nk >= 1 */
  int32_t d_qk;     /* query/key feature size */
  int32_t d_v;      /* value/output feature size */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
} blasst_shape_t;

/* Mask values written to mask_out. */
#define BLASST_TILE_DROPPED 0
#define BLASST_TILE_KEPT 1
#define BLASST_TILE_NOT_VISITED 2 /* no visible (row, key) pair: causally empty, or
                                     outside the block set in block-sparse mode */

/*
 * Prefill: out = skip-softmax attention of q against k, v.
 *
 *   q   [B, Hq,  Nq, d_qk]   (strides q_stride)
 *   k   [B, Hkv, Nk, d_qk]   (strides k_stride)
 *   v   [B, Hkv, Nk, d_v]    (strides v_stride)
 *   out [B, Hq,  Nq, d_v]    (strides o_stride), element type out_dtype
 *   mask_out  nullable, contiguous uint8 [B, Hq, ceil(Nq/br), ceil(Nk/bc)]:
 *             BLASST_TILE_* per (query tile, key tile)
 *   lse_out   nullable, contiguous float [B, Hq, Nq]: natural-log
 *             log-sum-exp of the scaled scores over the KEPT keys
 *   stats_out nullable, contiguous int64 [B, Hq, 2]: {visited key tiles,
 *             kept key tiles} summed over the head's query tiles
 *
 * Supported (else BLASST_E_UNSUPPORTED):
 *   BLASST_FP32, d_qk = d_v = 64,  br = 64,  bc = 64
 *   BLASST_BF16, d_qk = d_v = 128, br = 128, bc = 64
 */
blasst_status_t blasst_attn_prefill(const void* q, const void* k, const void* v, void* out,
                                    uint8_t* mask_out, float* lse_out, int64_t* stats_out,
                                    const blasst_shape_t* shape, blasst_dtype_t dtype,
                                    blasst_dtype_t out_dtype, float lambda, float scale,
                                    int causal, int br, int bc, void* stream);

/*
 * Block-sparse prefill: blasst_attn_prefill restricted to a caller-given set
 * of (query tile, key tile) blocks. Plain softmax attention computed inside a
 * selected block set is the final stage of block-sparse prefill methods (the
 * CRISP summary on rit.work, section "Что сделали"); block-sparse masks are
 * one of the mask kinds of the LongCA-bench post on denisavetisyan.com
 * (section "Сад Внимания: LongCA-bench и Стандартизация Оценки").
 *
 *   block_mask         DEVICE uint8 [B, Hq, ceil(Nq/br), ceil(Nk/bc)], owned
 *                      by the caller, read only: nonzero marks a block the
 *                      query tile may attend
 *   block_mask_stride  HOST int64[3]: element strides of block_mask's batch,
 *                      head and query-tile dimensions (>= 0; 0 broadcasts one
 *                      set over that dimension); key tiles are contiguous
 *   everything else    as for blasst_attn_prefill
 *
 * A (query, key) pair is visible when the causal rule allows it and its block
 * is in the set. The skip rule runs over the set's key tiles only, in
 * increasing order: the first of them that a query tile visits is always
 * kept, and the running max covers kept tiles of the set. Blocks outside the
 * set are reported BLASST_TILE_NOT_VISITED and never read. A query row that
 * sees no key at all gets a zero output row and lse -inf. With every block in
 * the set the result equals blasst_attn_prefill's.
 *
 * Supported (else BLASST_E_UNSUPPORTED): BLASST_BF16, d_qk = d_v = 128,
 * br = 128, bc = 64, ceil(Nk/64) <= 6144 (Nk <= 393216).
 * NULL block_mask_stride, or NULL block_mask for a call with query rows, is
 * BLASST_E_NULL; a negative stride is
 * BLASST_E_SHAPE.
 */
blasst_status_t blasst_attn_prefill_masked(const void* q, const void* k, const void* v,
                                           const uint8_t* block_mask,
                                           const int64_t block_mask_stride[3], void* out,
                                           uint8_t* mask_out, float* lse_out,
                                           int64_t* stats_out, const blasst_shape_t* shape,
                                           blasst_dtype_t dtype, blasst_dtype_t out_dtype,
                                           float lambda, float scale, int causal, int br, int bc,
                                           void* stream);

/*
 * MXFP4 quantization, the 4-bit format of the two-pass prefill's max
 * pre-pass (OCP Microscaling Formats (MX) Specification v1.0: FP4 E2M1
 * elements sharing one E8M0 scale per block of 32 consecutive features).
 * Per block: shared = floor(log2 max|x|) - 2, clamped to [-127, 127] (an
 * all-zero block takes -127); each element is x / 2^shared rounded to the
 * nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even code, larger values
 * clamped to 6), with the sign bit of x.
 *
 *   x         DEVICE bf16 [d0, d1, n, d], element strides x_stride[0..2]
 *             (HOST int64[3]), features contiguous; read only
 *   codes     DEVICE uint8 [d0, d1, n, d / 2], contiguous, written: feature 2j
 *             of a row in the low nibble of byte j; a code is sign << 3 |
 *             index of the magnitude in the list above
 *   scales    DEVICE uint8 [d0, d1, n, d / 32], contiguous, written: shared + 127
 *   stream    hipStream_t; asynchronous
 *
 * d must be a positive multiple of 32; x and codes 16-byte aligned, strides
 * multiples of 8 elements. Inputs must be finite. dtype must be BLASST_BF16.
 */
blasst_status_t blasst_quantize_mxfp4(const void* x, const int64_t x_stride[3], int32_t d0,
                                      int32_t d1, int32_t n, int32_t d, blasst_dtype_t dtype,
                                      uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Two-pass prefill. A reply in the digg thread "BLASST wins Best Paper at
 * MLSys 2026 ..." proposes a first pass that recomputes q.k in 4-bit only to
 * find the maxima, then gathering the kept blocks for the real computation.
 * Pass 1 quantizes q and k to MXFP4 (blasst_quantize_mxfp4, into the
 * workspace) and runs the skip rule of blasst_attn_prefill on the scores of
 * the quantized values (scale * q~.k~, same lambda, tiles and conventions),
 * which gives the tile map. Pass 2 computes exact softmax attention over the
 * map's kept tiles (the block-sparse prefill with lambda = 0 and the kept
 * tiles as the set). Decisions therefore follow the 4-bit scores and may
 * differ from blasst_attn_prefill's; the output is exact given the map.
 *
 *   q, k, v, out, lse_out   as for blasst_attn_prefill
 *   mask_out   nullable: the pass-1 map [B, Hq, ceil(Nq/br), ceil(Nk/bc)]
 *              (0 dropped, 1 kept, 2 not visited); when NULL the map lives in
 *              the workspace
 *   stats_out  nullable [B, Hq, 2] = {visited, kept} of the map
 *   workspace  DEVICE, 256-byte aligned, at least
 *              blasst_prefill_twopass_workspace_size bytes; holds the MXFP4
 *              copies of q and k and the map; its contents do not carry over
 *              between calls, and overlapping calls must not share it
 *
 * Supported (else BLASST_E_UNSUPPORTED): BLASST_BF16, d_qk = d_v = 128,
 * br = 128, bc = 64, ceil(Nk/64) <= 6144. Validation as for
 * blasst_attn_prefill_masked, plus BLASST_E_WORKSPACE.
 */
blasst_status_t blasst_attn_prefill_twopass(const void* q, const void* k, const void* v,
                                            void* out, uint8_t* mask_out, float* lse_out,
                                            int64_t* stats_out, const blasst_shape_t* shape,
                                            blasst_dtype_t dtype, blasst_dtype_t out_dtype,
                                            float lambda, float scale, int causal, int br, int bc,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * Workspace bytes blasst_attn_prefill_twopass needs for this shape. Validates
 * the size, dtype and tile combination and writes *bytes only on BLASST_OK.
 * Launches nothing.
 */
blasst_status_t blasst_prefill_twopass_workspace_size(const blasst_shape_t* shape,
                                                      blasst_dtype_t dtype, int causal, int br,
                                                      int bc, size_t* bytes);

/*
 * Prefill backward: gradients of a bf16 skip-softmax prefill with its tile
 * mask held fixed. Fine-tuning a model with the skip kernels in place improves
 * its quality (the BLASST post, paragraph beginning "Все изменения можно
 * делать без дообучения"); the keep/drop decisions are piecewise constant in
 * the inputs, so the gradient is that of softmax attention over the kept
 * tiles. With A = causal visibility AND the kept tiles of `mask`, and
 * P = exp(scale q.k - lse) on A (0 elsewhere):
 *   dv = P^T dout,  dP = dout v^T,  delta = rowsum(dout * out),
 *   dS = P (dP - delta),  dq = scale dS k,  dk = scale dS^T q,
 * dk and dv of a KV head summed over the query heads that read it.
 *
 *   q, k, v    the forward's inputs (bf16), strides as in the shape
 *   out        the forward's output, element type out_dtype, strides o_stride
 *   dout       gradient of the loss with respect to out, bf16, strides o_stride
 *   lse        the forward's lse_out, contiguous float [B, Hq, Nq] (a row with
 *              lse = -inf, one that saw no key, gets no gradient)
 *   mask       the forward's mask_out, contiguous uint8 [B, Hq, ceil(Nq/br),
 *              ceil(Nk/bc)]; only tiles marked BLASST_TILE_KEPT take part
 *   dq, dk, dv float outputs with the element strides of q, k and v; every
 *              element is written (rows of keys no query keeps get zeros)
 *   workspace  device memory of at least blasst_prefill_backward_workspace_size()
 *              bytes (B * Hq * Nq floats), 256-byte aligned, owned by the
 *              caller; contents on entry are ignored. Calls that overlap in
 *              time must not share it.
 *
 * Supported (else BLASST_E_UNSUPPORTED): BLASST_BF16, d_qk = d_v = 128,
 * br = 128, bc = 64, at most 6144 query tiles and 6144 key tiles, position
 * strides at most 2^24 elements. Any mask produced by blasst_attn_prefill or
 * blasst_attn_prefill_masked with these tiles is accepted.
 */
blasst_status_t blasst_attn_prefill_backward(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, const uint8_t* mask, float* dq, float* dk, float* dv,
    const blasst_shape_t* shape, blasst_dtype_t dtype, blasst_dtype_t out_dtype, float scale,
    int causal, int br, int bc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes blasst_attn_prefill_backward needs for this shape. Validates
 * like the call (sizes, dtype, supported combination) and writes *bytes only
 * on BLASST_OK. Launches nothing.
 */
blasst_status_t blasst_prefill_backward_workspace_size(const blasst_shape_t* shape,
                                                       blasst_dtype_t dtype, int causal, int br,
                                                       int bc, size_t* bytes);

/*
 * Decode: one query token per (batch, query head) against a contiguous KV
 * cache of len_kv positions (shape->len_q must be 1). Tile 0 is the cache's
 * first key tile and the running max is global along the whole cache, so the
 * mask does not depend on how the kernel splits the keys.
 *
 *   q       [B, Hq, d_qk]        (strides q_stride[0..1])
 *   k_cache [B, Hkv, Nk, d_qk]   (strides k_stride)
 *   v_cache [B, Hkv, Nk, d_v]    (strides v_stride), or NULL: the values are
 *           the first d_v features of each key (an MLA latent cache); then
 *           d_v < d_qk and v_stride is ignored
 *   out     [B, Hq, d_v]         (strides o_stride[0..1]), element type out_dtype
 *   mask_out  nullable, contiguous uint8 [B, Hq, ceil(Nk/bc)]
 *   lse_out   nullable, contiguous float [B, Hq]
 *   stats_out nullable, contiguous int64 [B, Hq, 3]: {visited key tiles, kept
 *             key tiles, V tiles read for this head's KV head}. A V tile is
 *             read when any query head sharing the KV head keeps it.
 *   workspace device memory of at least blasst_decode_workspace_size() bytes,
 *             256-byte aligned, owned by the caller; contents on entry are
 *             ignored and on return are undefined. May be NULL when that size
 *             is 0. Calls that overlap in time must not share a workspace.
 *
 * Supported (else BLASST_E_UNSUPPORTED), all BLASST_BF16 inputs with bc = 64:
 *   d_qk = d_v = 128 with a separate v_cache, heads_q / heads_kv <= 16.
 *           With batch * heads_kv >= 128 one workgroup walks each cache (no
 *           workspace). Below that the cache is split along its length over
 *           workgroups: a first pass stores the scores and tile maxima in the
 *           workspace, a second decides exactly from them, reads V for kept
 *           tiles only and writes per-split partials, and a log-sum-exp merge
 *           ends the call; the workspace grows with
 *           batch * heads_kv * ceil(Nk/64) * 256 * (heads_q/heads_kv) bytes;
 *   d_qk = 576, d_v = 512, v_cache NULL (latent cache), any heads_q / heads_kv.
 *           The cache is split along its length over workgroups; the
 *           workspace holds the tile maxima, the per-split partial outputs
 *           and their log-sum-exp statistics, merged at the end. It grows
 *           with B * Hq * (ceil(Nk/64) + 2 KB per split).
 */
blasst_status_t blasst_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                   void* out, uint8_t* mask_out, float* lse_out,
                                   int64_t* stats_out, const blasst_shape_t* shape,
                                   blasst_dtype_t dtype, blasst_dtype_t out_dtype, float lambda,
                                   float scale, int bc, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory or
 * take a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, validation, kernels and
 * results as blasst_attn_decode, without the workspace: the scratch the
 * latent-cache decode needs (tile maxima, split partials) lives in one static
 * device array per GPU inside the library, 64 MiB, reserved on each GPU the
 * library runs on until the process ends. The call allocates nothing. A shape
 * whose scratch (blasst_attn_decode_workspace_size) exceeds 64 MiB returns
 * BLASST_E_UNSUPPORTED. Every call on one GPU uses that GPU's array: calls that
 * overlap in time on one GPU (concurrent streams or host threads) race and
 * must be serialised by the caller. Nothing in the array needs to start at any
 * value; a call's contents are dead once it completes.
 */
blasst_status_t blasst_attn_decode_noalloc(const void* q, const void* k_cache,
                                           const void* v_cache, void* out, uint8_t* mask_out,
                                           float* lse_out, int64_t* stats_out,
                                           const blasst_shape_t* shape, blasst_dtype_t dtype,
                                           blasst_dtype_t out_dtype, float lambda, float scale,
                                           int bc, void* stream);

/*
 * Workspace bytes blasst_attn_decode needs for this shape, dtype, cache kind
 * (has_v_cache = 0 for a latent cache) and tile size; 0 when none is needed.
 * Validates like blasst_attn_decode (sizes, dtype, supported combination) and
 * writes *bytes only on BLASST_OK. Launches nothing.
 */
blasst_status_t blasst_decode_workspace_size(const blasst_shape_t* shape, blasst_dtype_t dtype,
                                             int has_v_cache, int bc, size_t* bytes);

/*
 * The same query in the form the hot-path contract names: the cache kind is
 * taken from the sizes (d_v < d_qk is a latent cache whose values are the
 * first d_v features of each key, v_cache NULL; otherwise a separate v_cache).
 * Returns the workspace bytes blasst_attn_decode needs (0 when none), or
 * SIZE_MAX when the shape, dtype or tile size has no decode kernel or shape is
 * NULL; blasst_last_error() then says why. Launches nothing.
 */
size_t blasst_attn_decode_workspace_size(const blasst_shape_t* shape, blasst_dtype_t dtype,
                                         int bc);

/* Static text for a status code. */
const char* blasst_status_string(blasst_status_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char* blasst_last_error(void);

/* BLASST_VERSION of the loaded library. */
int blasst_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLASST_H */
