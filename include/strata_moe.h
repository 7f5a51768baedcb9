/*
 * strata_moe.h -- C ABI of the routed-expert MoE layer on MI355X (gfx950).
 *
 * One MoE layer of a 48-layer, 512-expert, top-10 model with H = 2560 and
 * FF = 640.  The pages this follows are cited by title and section:
 *
 *  [SRC]  "Strata in the source: one verify window, three workers and a cache
 *          that learns" (ai.thesatyajit.com).
 *  [ZW]   "MoE 遇上消费级显卡动态路由专家权重12GB 怎么装下 125B 不爆显存"
 *          (zwxr.cn), the passage that follows one token through one layer
 *          (算 logits / 选 top-10 / 命中与未命中拆分 / Combine).
 *  [MY]   the momoyeyu.github.io Strata explainer (ai-infra-strata),
 *          section 提示词处理 (prompt processing).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless stated otherwise, row-major, owned by
 *    the caller.  The library never allocates or frees inside these calls and
 *    keeps no pointer after it returns; enqueued kernels use the buffers until
 *    the stream passes them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *  - Arguments are validated on the host before anything is enqueued: a call
 *    that returns an error enqueued nothing.  No call synchronises the host,
 *    reads device memory from the host, or uses memset, so calls may be
 *    captured into a HIP graph -- except strata_moe_read_status and
 *    strata_moe_verify_blobs, a diagnostic and a load-time check that
 *    synchronise their stream and say so below.  Device faults surface at
 *    the caller's next synchronisation.
 *  - Results are deterministic: the same inputs and T give the same bits
 *    (no floating-point atomics anywhere).
 *  - Alignment: `blobs` and `ws` 256 bytes; x, y, out and router 16 bytes;
 *    every other array 4 bytes.  A violation returns STRATA_E_ALIGN.
 */
#ifndef STRATA_MOE_H_INCLUDED
#define STRATA_MOE_H_INCLUDED

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define STRATA_API __attribute__((visibility("default")))
#else
#define STRATA_API
#endif

/* Layer geometry, fixed at compile time ([SRC] "The byte budget, in code";
 * [ZW] 48 x 512 experts, top-10). */
#define STRATA_MOE_H 2560      /* hidden size */
#define STRATA_MOE_FF 640      /* expert intermediate width */
#define STRATA_MOE_E 512       /* routed experts per layer */
#define STRATA_MOE_K 10        /* experts per token */
#define STRATA_MOE_QK 64       /* weights per Q2_0 block */
#define STRATA_MOE_BB 18       /* bytes per Q2_0 block: fp16 scale, 16 code bytes */
#define STRATA_MOE_BLOB 1382400 /* bytes per expert blob: gate, up, down */
#define STRATA_MOE_T_MAX 8192  /* largest token count per call (one prefill chunk) */
#define STRATA_LOOKAHEAD_T_MAX 8 /* largest token count of strata_moe_layer_lookahead */
#define STRATA_STATIC_T_MAX 64   /* largest token count of strata_moe_layer_static */

/* Status codes. */
#define STRATA_OK 0
#define STRATA_E_ARG (-1)       /* NULL pointer or bad flag */
#define STRATA_E_SHAPE (-2)     /* T outside 1..STRATA_MOE_T_MAX */
#define STRATA_E_WORKSPACE (-3) /* workspace missing or smaller than required */
#define STRATA_E_HIP (-4)       /* the HIP runtime reported a launch error */
#define STRATA_E_ALIGN (-5)     /* a pointer breaks the alignment rule above */
#define STRATA_E_CORRUPT (-6)   /* strata_moe_verify_blobs: a blob differs from its checksum */

/* Bits of a workspace's status word (see strata_moe_read_status). */
#define STRATA_STATUS_WAIT_TIMEOUT 1 /* a decode experts wait gave up: outputs of that call are NaN */

/* Flags. */
#define STRATA_RMSNORM 1  /* normalise x first: x / sqrt(mean(x^2) + 1e-6), unit gain */
#define STRATA_RESIDUAL 2 /* combine adds into its output (x += y) instead of storing */
#define STRATA_INT8 4     /* experts and layer calls with T > 16: the integer variant (below) */

/* Bytes of one Q2_0 expert blob (1,382,400): the gate [FF][H], up [FF][H] and
 * down [H][FF] matrices in that order, each row a run of 18-byte blocks along
 * the matrix's input dimension; a block is a little-endian fp16 scale d
 * followed by 16 bytes holding 64 two-bit codes, code i at bits 2i..2i+1 of
 * the little-endian 128-bit field; code c means weight (c - 1) * d
 * ([SRC] "The byte budget, in code" and "The CPU kernels").  A layer's store
 * is 512 blobs back to back, expert e at e * STRATA_MOE_BLOB. */
STRATA_API size_t strata_moe_blob_bytes(void);

/* Workspace bytes a call with T tokens needs (0 if T is out of range).  Every
 * entry point below that takes `ws` needs at least this much for its T. */
STRATA_API size_t strata_moe_workspace_bytes(int T);

/* Router ([ZW] 算 logits, 选 top-10): per token, logits = xhat . R^T (+ bias)
 * with R in bf16 and fp32 accumulation, softmax over all 512 experts, a stable
 * descending sort (equal probabilities keep the lower expert id first), the
 * first 10 ids, and weights p_k / max(sum of the 10 p, 2^-14).
 *   x      [T][H] fp32 activations; xhat = x, or RMSNorm(x) with STRATA_RMSNORM.
 *   router [E][H] bf16 bit patterns.
 *   bias   [E] fp32 added to the logits before the softmax, or NULL.
 *   ids    [T][K] int32 out: expert ids in descending-weight order.
 *   w      [T][K] fp32 out: renormalised weights (sum 1 per token).
 * Returns STRATA_OK or an error code. */
STRATA_API int strata_moe_route(const float *x, int T, const uint16_t *router, const float *bias,
                     int flags, int32_t *ids, float *w, void *ws, size_t ws_bytes,
                     void *stream);

/* Token -> expert grouping ([MY] 提示词处理: collect tokens per expert so one
 * weight read serves every token routed to it; [SRC] "The plan: three
 * destinations per expert": a window's routed ids are deduplicated first).
 *   ids     [T][K] int32 in, values in 0..511 (others are dropped).
 *   offsets [E+1] int32 out: exclusive prefix sum of per-expert slot counts.
 *   slots   [T*K] int32 out: flat slot ids t*K+k ordered by expert, stable
 *           (ascending slot id within an expert).
 *   active  [1+E] int32 out: active[0] = number of experts with at least one
 *           slot, active[1..] those expert ids in ascending order. */
STRATA_API int strata_moe_group(const int32_t *ids, int T, int32_t *offsets, int32_t *slots,
                     int32_t *active, void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs ([SRC] "The byte budget, in code": each expert is a gate, an up
 * and a down matrix of 2,560 x 640 Q2_0 weights; [MY] 提示词处理: a chunk's
 * tokens are grouped per expert and each expert's weights are dequantised and
 * multiplied once for all of its tokens).  The expert function is SwiGLU:
 * for every grouped slot s = t*K+k of expert e,
 *   out[s] = W_d (silu(W_g xhat_t) * (W_u xhat_t)),  silu(z) = z / (1 + e^-z),
 * reading each active expert's blob once for all of its tokens.
 *   x       [T][H] fp32; xhat as in strata_moe_route (STRATA_RMSNORM).
 *   blobs   [E][BLOB] bytes, one layer's store (256-byte aligned).
 *   offsets, slots, active: as written by strata_moe_group for the same T.
 *   out     [T*K][H] fp32 out, unweighted expert outputs by flat slot id.
 * Decode-sized T (T <= 16) uses one bandwidth-bound kernel of integer dot
 * products: x as 16-bit integers per 64-value block and h per 16-value
 * segment, against the exact 2-bit codes, with exact int32 block sums and
 * fp32 across blocks; larger T uses fp16 MFMA grouped GEMMs with exactly
 * dequantised weights and fp32 accumulation.  For T > 16 the fp16
 * activations carry an exact per-token power-of-two scale (the token's
 * largest |xhat| maps into [2^12, 2^13)), and h one that follows the square
 * of the input's magnitude outside [1, 8), so inputs of any magnitude stay
 * in fp16's range; an h value whose magnitude exceeds 65504 times that
 * scale would overflow to inf.
 * With STRATA_INT8 and T > 16, the integer variant of [SRC] "The CPU
 * kernels" runs instead: xhat and h as int8 per 64-value block (scale
 * max|v| / 127), the raw codes on int8 MFMA with the code offset removed by
 * the block's -(sum q), fp32 across blocks.  Its results differ from the
 * exact layer by the int8 rounding of the activations (about 1e-2 of max|y|;
 * see the parity tests), which the fp16 path does not have. */
STRATA_API int strata_moe_experts(const float *x, int T, const uint8_t *blobs, const int32_t *offsets,
                       const int32_t *slots, const int32_t *active, int flags, float *out,
                       void *ws, size_t ws_bytes, void *stream);

/* Weighted combine ([ZW] Combine: sum of w[i] * parts[i]):
 *   y[t] = sum over k = 0..9 in routing order of w[t][k] * out[t*K+k];
 * with STRATA_RESIDUAL, y[t] += that sum instead.
 *   out [T*K][H] fp32 in, w [T][K] fp32 in, y [T][H] fp32 out (or in/out). */
STRATA_API int strata_moe_combine(const float *out, const float *w, int T, int flags, float *y,
                       void *stream);

/* The whole layer in one call ([ZW], the passage that follows one token
 * through a layer: logits, top-10, the experts, then one weighted Combine):
 * route -> group -> experts -> combine.
 *   x      [T][H] fp32 in; with STRATA_RESIDUAL also out (x += layer output).
 *   y      [T][H] fp32 out (layer output without residual), or NULL; must not
 *          be NULL unless STRATA_RESIDUAL is set.
 *   ids, w [T][K] out, or NULL to keep them in the workspace.
 * Other arguments as above (flags: STRATA_RMSNORM, STRATA_RESIDUAL,
 * STRATA_INT8).  Results equal the four-call composition. */
STRATA_API int strata_moe_layer(float *x, int T, const uint16_t *router, const float *bias,
                     const uint8_t *blobs, int flags, float *y, int32_t *ids, float *w,
                     void *ws, size_t ws_bytes, void *stream);

/* The layer with a router lookahead ([ZW], the passage on prefetching and
 * warm-up: the next layer's router is run on this layer's MoE input, because
 * the residual stream changes little between adjacent layers, to predict the
 * next layer's experts and warm their bytes without changing any result).
 * Does what strata_moe_layer does with the first nine arguments, with
 * bitwise the same outputs, and also:
 *  - routes the same normalised input through router_next [E][H] bf16 (plus
 *    bias_next [E] fp32, or NULL) to that layer's ten ids per token, written
 *    to pred_ids [T][K] int32 (or kept in the workspace when NULL);
 *  - reads the predicted experts' blobs in blobs_next (the next layer's store,
 *    [E][BLOB], 256-byte aligned) once, line by line, in the experts
 *    launch's tail, so that they sit in the memory-side cache when the next
 *    layer runs;
 *  - for T = 1, takes hint_ids [1][K] int32 (device memory, or NULL): the ids
 *    this token is expected to route to, normally the previous lookahead
 *    call's pred_ids.  The gate/up rows of the hinted experts are requested
 *    before the token's own routing has finished, and used for the heads
 *    whose expert they are; heads no hint names are read after the routing.
 *    Any values are allowed (ids outside 0..E-1 and repeats are ignored).
 *    Ignored for T > 1.
 * Nothing is written to blobs_next, and no result depends on blobs_next or
 * on hint_ids.
 * T must be 1..STRATA_LOOKAHEAD_T_MAX (decode); other T return STRATA_E_SHAPE.
 * router_next and blobs_next must not be NULL (STRATA_E_ARG). */
STRATA_API int strata_moe_layer_lookahead(float *x, int T, const uint16_t *router,
                               const float *bias, const uint8_t *blobs, int flags, float *y,
                               int32_t *ids, float *w, const uint16_t *router_next,
                               const float *bias_next, const uint8_t *blobs_next,
                               int32_t *pred_ids, const int32_t *hint_ids, void *ws,
                               size_t ws_bytes, void *stream);

/* strata_moe_layer for callers that cannot allocate (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the same
 * arguments without `ws` / `ws_bytes`, and bitwise the same results.  Its
 * workspace is a static device array of 10 MiB per GPU, part of the library's
 * code object (it stays allocated until the process ends); its address is
 * looked up once per device on the first call made with that device
 * current.  No call allocates or frees anything.
 *  - T must be 1..STRATA_STATIC_T_MAX (64); larger T return STRATA_E_SHAPE
 *    and enqueue nothing.
 *  - Every call on one GPU uses the same array, which keeps the last call's
 *    contents: calls that overlap on one GPU (other streams, other threads)
 *    race and must be serialised by the caller.  Each call clears what it
 *    needs cleared itself.
 *  - The array's first 4 bytes are its status word (see below); it is zero
 *    when the library is loaded and is never cleared by the library.
 *  - STRATA_E_HIP if the array's address cannot be obtained. */
STRATA_API int strata_moe_layer_static(float *x, int T, const uint16_t *router, const float *bias,
                                       const uint8_t *blobs, int flags, float *y, int32_t *ids,
                                       float *w, void *stream);

/* Measurement hook (not part of the layer's math): arms the next
 * strata_moe_experts or strata_moe_layer call made by this host thread to
 * launch its dominant kernel with the HIP events `start` and `stop`
 * (hipEvent_t) attached to the dispatch itself (hipExtLaunchKernel), so that
 * hipEventElapsedTime(start, stop) is that kernel's own duration.  The kernel
 * is, for decode-sized T, the fused experts kernel (gate/up, down and, in the
 * layer call, the combine), and for larger T the gate/up GEMM.  A layer call
 * of 1..3 tokens runs its experts as two launches (gate/up, then down with the
 * combine); there `start` is on the first and `stop` on the second, and the
 * first launch also routes the tokens.
 * The hook is used by one call and disarmed.  Events are the caller's; pass both NULL to
 * disarm.  Returns STRATA_E_ARG if only one is NULL.  Not for use under graph
 * capture. */
STRATA_API int strata_moe_time_next_kernel(void *start, void *stop);

/* Status word.  The first 4 bytes of every workspace hold a status word that
 * the kernels OR STRATA_STATUS_* bits into and never clear.  The decode-sized
 * experts kernel (T <= 16) has one wait: a unit's down part waits for the
 * gate/up results of its expert's other units, which the dispatch order
 * guarantees to come (workgroups start in index order on each XCD).  The wait
 * is bounded; if it gives up, the outputs that depended on it are set to NaN
 * and STRATA_STATUS_WAIT_TIMEOUT is set, so such a failure never passes as a
 * result.  A fresh workspace must have its status word zeroed once (the
 * Python binding's workspace() does; or call strata_moe_clear_status).
 *
 * strata_moe_read_status: synchronises `stream`, then copies the status word
 * of `ws` (at least 256 bytes, 256-byte aligned) to *bits (host memory).  A
 * diagnostic: not for use under graph capture.  Returns STRATA_OK,
 * STRATA_E_ARG, STRATA_E_WORKSPACE, STRATA_E_ALIGN or STRATA_E_HIP. */
STRATA_API int strata_moe_read_status(const void *ws, size_t ws_bytes, int32_t *bits,
                                      void *stream);

/* Enqueues on `stream` a kernel that sets the status word of `ws` to 0
 * (capturable: no memset). */
STRATA_API int strata_moe_clear_status(void *ws, size_t ws_bytes, void *stream);

/* Bound of the decode experts kernel's wait, in polls of the expert's counter
 * (each about 0.2-1 us); 0 restores the default of 2^18, negative values
 * return STRATA_E_ARG.  Applies to launches made after the call, from any
 * thread.  Meant for tests of the failure path (a bound of 1 makes most waits
 * give up at once, so every kernel still ends). */
STRATA_API int strata_moe_set_wait_limit(int polls);

/* Blob-store integrity ([ZW], the passage on how the design differs from
 * static offload, third point: every cache slot is read back after it is
 * filled and a mismatch refuses to run).  Here the whole store sits in HBM,
 * filled once, and each blob gets a 64-bit checksum:
 *   checksum = sum over the blob's little-endian 64-bit words w_j
 *              (j = 0 .. STRATA_MOE_BLOB / 8 - 1) of
 *              mix(w_j + (j + 1) * 0x9E3779B97F4A7C15) mod 2^64,
 * mix being SplitMix64's output function (z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 * z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31).
 *
 * strata_moe_blob_checksums: enqueues the checksums of nblobs consecutive
 * device blobs (blobs 256-byte aligned, nblobs * STRATA_MOE_BLOB bytes) into
 * sums [nblobs] (device, 8-byte aligned).  Capturable.  STRATA_E_SHAPE for
 * nblobs outside 1..STRATA_MOE_CHECK_BLOBS_MAX.
 *
 * strata_moe_blob_checksum_host: the checksum of one blob in HOST memory
 * (STRATA_MOE_BLOB bytes), computed on the CPU, for the expected values of a
 * store at load time; 0 for a NULL pointer.
 *
 * strata_moe_verify_blobs: the checksums of nblobs device blobs (into the
 * caller's device scratch sums [nblobs]) compared with expected [nblobs] in
 * HOST memory.  Synchronises `stream` (a load-time check, not for graph
 * capture).  Returns STRATA_OK with *first_bad = -1, or STRATA_E_CORRUPT with
 * *first_bad (host) the lowest index whose checksum differs; the argument
 * errors of strata_moe_blob_checksums, or STRATA_E_HIP. */
#define STRATA_MOE_CHECK_BLOBS_MAX (1 << 24)
STRATA_API int strata_moe_blob_checksums(const uint8_t *blobs, int64_t nblobs, uint64_t *sums,
                                         void *stream);
STRATA_API uint64_t strata_moe_blob_checksum_host(const uint8_t *blob);
STRATA_API int strata_moe_verify_blobs(const uint8_t *blobs, int64_t nblobs,
                                       const uint64_t *expected, uint64_t *sums,
                                       int64_t *first_bad, void *stream);

/* Human-readable text of a status code (static storage). */
STRATA_API const char *strata_moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_MOE_H_INCLUDED */
