/*
 * triroute.h -- C ABI of the MI355X (gfx950) library for TriRoute's inference hot path:
 * routed attention over a KV cache whose precision varies per token.
 *
 * Source of the method: "TriRoute: Unified Learned Routing for Joint Adaptive Attention,
 * Experts, and KV-Cache Allocation", paper-review page on xllm-io.github.io:
 *   - Eq. (4), "(C) KV-cache bit width": each token's K and V are quantized asymmetrically,
 *     per token, at a width b in {2, 4, 8, 16} chosen by the controller;
 *     s = (max - min) / (2^b - 1), z = min, code = round((x - z) / s); b = 16 is native storage.
 *   - Eq. (2), "(A) attention resolution": each (query token, head) runs in one of three
 *     modes -- skip (output 0), local-w (keys t-w .. t) or full causal (keys <= t).
 *   - the inference paragraph after Algorithm 1: hard decisions, skipped work never
 *     materialized, each token's KV stored at its chosen width, one left-to-right pass,
 *     compatible with batching and KV paging.
 * The routing decisions (mode per query head, b per token) are inputs to every attention call,
 * as in the page's problem statement.  tr_controller_route (below) produces them on the device
 * from the residual stream with the page's controller at inference (Eq. (5), Eq. (11), hard
 * argmax), given its weights.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HIP device memory), owned by the caller, unless
 *     a comment says otherwise.  bf16 tensors are passed as raw 16-bit patterns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call is
 *     asynchronous on that stream; the caller keeps the inputs alive until the stream reaches
 *     the call.  Calls on one cache must be ordered (one stream, or caller-side events).
 *   - Host-side argument checks run first and synchronously; on failure the call returns an
 *     error and launches nothing.  Element values that only the device sees (a width not in
 *     {2,4,8,16}, a mode > 2) and pool exhaustion set sticky flags in the cache, read by
 *     tr_kv_cache_status(); outputs touched by a bad element are unspecified.
 *   - No call throws; no call allocates except tr_kv_cache_alloc.
 *   - Inputs must be finite; for every quantized group max - min must be finite in fp32.
 *     tr_routed_attn_prefill also bounds the V values it reads (see there).
 *   - Quantization is bit-exact: s = fl32(fl32(max - min) / (2^b - 1)) with a correctly
 *     rounded divide, z = min (+0 for a zero minimum), code = rint(fl32(fl32(x - z) / s)),
 *     codes 0 for a constant group.  Attention accumulates in fp32 and writes bf16 (RNE).
 *   - Local windows are the inclusive range [max(0, t - w), t] (w + 1 keys); scores are
 *     scaled by 1/sqrt(head_dim); the query attends to its own freshly written K/V.
 */
#ifndef TRIROUTE_H_
#define TRIROUTE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TR_OK = 0,
  TR_ERR_INVALID_ARG = 1,   /* a host-checked argument is out of range or NULL */
  TR_ERR_CAPACITY = 2,      /* the write would exceed the per-sequence capacity max_tokens */
  TR_ERR_OUT_OF_PAGES = 3,  /* sticky: the page pool ran out during a write */
  TR_ERR_HIP = 4,           /* a HIP runtime call failed (allocation, launch, copy) */
  TR_ERR_UNSUPPORTED = 5,   /* a valid but unsupported shape (head_dim not 64/128, ...) */
  TR_ERR_BAD_VALUE = 6,     /* sticky: a bits or mode element outside its domain was seen */
  TR_ERR_RANGE = 7,         /* sticky: a value outside fp16's range (prefill's v_hat, the expert FFN) */
  TR_ERR_SCRATCH = 8        /* tr_routed_attn_decode_noalloc: the call needs more scratch than
                               its fixed array holds (nothing launched) */
} tr_status;

/* Attention modes of Eq. (2): one uint8 per (sequence, query token, head). */
enum { TR_MODE_SKIP = 0, TR_MODE_LOCAL = 1, TR_MODE_FULL = 2 };

/* Cache shape.  Host struct, read only during tr_kv_cache_alloc. */
typedef struct {
  int32_t num_layers;       /* >= 1 */
  int32_t batch;            /* sequences per layer, >= 1 */
  int32_t num_heads;        /* KV heads, >= 1 (the heads the cache stores) */
  int32_t head_dim;         /* 64 or 128 */
  int32_t max_tokens;       /* per-sequence capacity in positions, >= 1; at most
                               2^30 / head_dim (TR_ERR_UNSUPPORTED beyond) */
  int32_t page_code_bytes;  /* K (and V) code bytes of one head in one page; 0 -> 4096.
                               A power of two in [1024, 65536].  A page of width b holds
                               page_code_bytes * 8 / (head_dim * b) tokens. */
  int64_t pool_pages;       /* pages in the pool; 0 -> enough for any mix of widths */
  int32_t num_query_heads;  /* query heads of the attention calls: 0 -> num_heads (multi-head
                               attention), else a multiple of num_heads (grouped-query attention:
                               query head h reads KV head h / (num_query_heads / num_heads); the
                               review page's experimental setup, section 5, uses H_kv = H/4) */
  int32_t prefill_tokens;   /* scratch of tr_routed_attn_prefill: a prefill call may reach
                               positions up to prefill_tokens (len + T <= prefill_tokens).
                               0 -> max_tokens; -1 -> none (a decode-only cache: no prefill
                               scratch is allocated and tr_routed_attn_prefill returns
                               TR_ERR_UNSUPPORTED); else 1 .. max_tokens.  The scratch grows
                               with it: per (sequence, KV head) 4 * head_dim + 8 bytes per
                               position, plus per (sequence, query head) 4 bytes per position
                               and 16 partial tiles of 128 x (head_dim + 4) floats. */
} tr_kv_cache_desc;

/* Opaque cache: per (layer, sequence, width class) a stream of pages of the pool, fp32
 * (scale, zero) side arrays inside each page, per-position width-class prefix counts, and the
 * scratch buffers of the attention calls.  Owned by the library. */
typedef struct tr_kv_cache tr_kv_cache;

/* Allocate and zero a cache (device memory via hipMalloc, on the current device).
 * *out receives the handle; nothing is allocated on error.  Every field of the descriptor is
 * read, so zero-initialize it (0 picks each field's default). */
tr_status tr_kv_cache_alloc(const tr_kv_cache_desc* desc, tr_kv_cache** out);

/* Free every device buffer of the cache.  Synchronizes the device first.  NULL is a no-op. */
tr_status tr_kv_cache_free(tr_kv_cache* cache);

/* Empty every layer (lengths 0, all pages returned, sticky flags cleared), on `stream`. */
tr_status tr_kv_cache_reset(tr_kv_cache* cache, void* stream);

/* Roll `layer` back to its first new_len positions (0 <= new_len <= length), e.g. to discard
 * rejected speculative tokens.  Host-side only; the pages of the dropped positions stay
 * attached to their class streams and are reused by the next write. */
tr_status tr_kv_cache_truncate(tr_kv_cache* cache, int32_t layer, int32_t new_len);

/* Tokens written so far to `layer` (the same for every sequence).  -1 on a bad argument. */
int32_t tr_kv_cache_length(const tr_kv_cache* cache, int32_t layer);

/* Eq. (4) write: append n_new tokens to every sequence of `layer` at positions
 * len .. len + n_new - 1, each quantized at its own width.
 *   k, v:  bf16 [batch, n_new, num_heads, head_dim], row-major
 *   bits:  uint8 [batch, n_new], values in {2, 4, 8, 16}; one width per token, shared by the
 *          token's K, V and all heads (the page charges 2 * d_kv * b bits per token).
 * Each (token, head) K vector and V vector is one quantization group of head_dim values. */
tr_status tr_kv_quantize_write(tr_kv_cache* cache, int32_t layer, const void* k, const void* v,
                               const uint8_t* bits, int32_t n_new, void* stream);

/* Eq. (2) decode: one query per sequence at position t = len - 1 (its K/V must already be
 * written with tr_kv_quantize_write), attending in its per-head mode to the cached K/V.
 *   q:    bf16 [batch, num_query_heads, head_dim]
 *   mode: uint8 [batch, num_query_heads] (TR_MODE_*)
 *   window: w >= 0 for local heads
 *   out:  bf16 [batch, num_query_heads, head_dim]; skip heads get zeros */
tr_status tr_routed_attn_decode(tr_kv_cache* cache, int32_t layer, const void* q, const uint8_t* mode,
                                int32_t window, void* out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): tr_routed_attn_decode with every argument and result
 * the same, whose split-K partial results go to a fixed 8 MiB array in the library's device
 * memory (one per GPU, held until the process ends) instead of the cache's scratch.  It calls
 * no hipMalloc, hipFree or other allocating routine and records no profiling events.  The
 * partials of one call take B * num_query_heads * chunks * (head_dim + 2) * 4 bytes; the call
 * picks the chunk count as the plain entry point does, lowered to what fits, and returns
 * TR_ERR_SCRATCH (launching nothing) when even the fewest chunks a full window allows (windows
 * split into chunks of at most 512 positions) do not fit.  Calls on one GPU share the array:
 * two calls whose executions overlap on one GPU (different streams without ordering) race and
 * give unspecified results; calls ordered on one stream are safe.  Nothing in the array needs
 * to start at zero (every chunk writes its own record before the merge reads it). */
tr_status tr_routed_attn_decode_noalloc(tr_kv_cache* cache, int32_t layer, const void* q, const uint8_t* mode,
                                        int32_t window, void* out, void* stream);

/* Prefill: write T new tokens with Eq. (4), then run Eq. (2) for all T queries (causal, each
 * query at its own position len + i, reading the cache just written).
 *   q:    bf16 [batch, T, num_query_heads, head_dim]; k, v: bf16 [batch, T, num_heads, head_dim]
 *   bits: uint8 [batch, T];  mode: uint8 [batch, T, num_query_heads]
 *   out:  bf16 [batch, T, num_query_heads, head_dim]
 * Range: the prefill attention's PV product takes the stored values v_hat = s * c + z (the raw
 * value for b = 16) in fp16, so every V value the call reads -- its own tokens' and, for a call
 * that continues a sequence, the earlier positions' -- must satisfy |v_hat| < 65504.  V inputs
 * with every |v| <= 65280 (the largest bf16 below 65504) always do (v_hat stays within its
 * group's [min, max] up to 2^-22 relative).  A larger value sets the sticky TR_ERR_RANGE flag
 * (tr_kv_cache_status) and leaves the call's outputs unspecified; the cache contents are written
 * exactly as tr_kv_quantize_write would write them, and decode, which dequantizes in fp32, has no
 * such limit. */
tr_status tr_routed_attn_prefill(tr_kv_cache* cache, int32_t layer, const void* q, const void* k,
                                 const void* v, const uint8_t* bits, const uint8_t* mode, int32_t T,
                                 int32_t window, void* out, void* stream);

/* Diagnostic read-back of positions tok0 .. tok0 + n - 1 of every sequence of `layer`, in
 * position order, into caller device buffers:
 *   codes: uint16 [batch, n, 2, num_heads, head_dim]  (index 2: 0 = K, 1 = V); b < 16: the
 *          code; b = 16: the stored bf16 bits
 *   scale, zero: float [batch, n, 2, num_heads]; b = 16 tokens read (1, 0)
 *   bits: uint8 [batch, n] */
tr_status tr_kv_cache_export(const tr_kv_cache* cache, int32_t layer, int32_t tok0, int32_t n,
                             uint16_t* codes, float* scale, float* zero, uint8_t* bits, void* stream);

/* Synchronize `stream` and report the sticky device flags: TR_ERR_OUT_OF_PAGES, then
 * TR_ERR_BAD_VALUE, then TR_ERR_RANGE, else TR_OK. */
tr_status tr_kv_cache_status(tr_kv_cache* cache, void* stream);

/* Pages taken from the pool so far (synchronizes `stream`).  -1 on error. */
int64_t tr_kv_cache_pages_used(tr_kv_cache* cache, void* stream);

/* Diagnostics: the decode split-K.  Decode splits every attended window into position chunks
 * (each chunk one work item, the chunks merged by a log-sum-exp combine); by default the library
 * picks the count from the batch, heads and context.  n >= 1 forces n chunks over a full window
 * [0, t] (chunk length ceil((t + 1) / n); a local window gets as many chunks of that length as it
 * needs; n is capped at t + 1), n = 0 restores the automatic choice.  A later decode call returns
 * TR_ERR_UNSUPPORTED, and launches nothing, if the forced chunks would exceed a work item's limit
 * of 512 positions.  n must lie in [0, 64] (TR_ERR_INVALID_ARG otherwise).  Host-side only; the
 * output is the same up to fp32 reduction order for every n. */
tr_status tr_kv_cache_set_decode_chunks(tr_kv_cache* cache, int32_t n);

/* Diagnostics: while enabled, the library's kernel launches on this cache are bracketed by HIP
 * events on the call's stream.  tr_profile_read synchronizes on them, returns per kernel family
 * the number of launches and their summed duration in milliseconds since the last read, and
 * clears the record.  Families (array index): 0 quantize-write (slot assignment + quantize),
 * 1 decode split-K, 2 decode combine, 3 prefill preparation (row compaction, work units, the
 * slot assignment of a prefill call, and dense staging of earlier positions), 4 prefill attention,
 * 5 prefill merge of key-split tiles (and the zeros of skip rows).
 * launches and total_ms are HOST arrays of 6 elements. */
tr_status tr_profile_enable(tr_kv_cache* cache, int32_t enable);
tr_status tr_profile_read(tr_kv_cache* cache, int64_t* launches, double* total_ms);

/* Weights of the routing controller for one layer (TriRoute review page, "core formulas" item 5,
 * Eq. (5): a shared trunk maps [Norm(x_t); psi_t] to h_t in R^d_r, RMSNorm, then one linear head
 * per axis; item 10, Eq. (11): per-axis whitening with frozen statistics).  Host struct holding
 * DEVICE pointers; read during the call only.  The trunk is Linear(d + d_side -> 128) with bias,
 * SiLU, Linear(128 -> 128) with bias; Norm and RMSNorm have unit gain and eps 1e-6; the
 * whitening is (hhat - mu) / (sigma + 1e-5); the heads have no bias.
 *   w1       bf16  layer 1, residual part, PACKED by tr_controller_pack_w1 from [128][d] (out x
 *            in, row-major) -- d * 128 values in the matrix-core operand order
 *   w1_side  float [128][d_side]        layer 1, side-feature part (out x in); NULL if d_side = 0
 *   b1, b2   float [128]
 *   w2       float [128][128]           layer 2, stored in x out (element [i][o])
 *   mu_a, sigma_a, mu_b, sigma_b  float [128]   Eq. (11) statistics, attention / bit axis
 *   w_a      float [128][3 * heads]     attention head, in x out; head h's logits are columns
 *                                       3h (skip), 3h + 1 (local), 3h + 2 (full)
 *   w_b      float [128][4]             bit head, in x out; columns b = 2, 4, 8, 16
 * workspace (optional): DEVICE scratch of workspace_bytes >= tr_controller_workspace_bytes(d),
 * 16-byte aligned, caller owned, or NULL.  With it, calls of up to 256 tokens (a decode step)
 * spread the first layer over (tokens / 32 rounded up) x 4 x ceil(d / 256) workgroups and finish
 * each token in a workgroup of its own (two launches); without it, and for larger calls, one
 * workgroup handles 32 tokens.  Calls that share a workspace must be ordered (one stream); its
 * contents need no initialization and are not kept between calls. */
typedef struct {
  int32_t d;                /* model width: a multiple of 64, 64 .. 16384 */
  int32_t d_side;           /* side features per token, 0 .. 32 */
  int32_t d_r;              /* trunk width: must be 128 (the page's d_r) */
  int32_t heads;            /* attention heads routed per token, 1 .. 64 */
  const void* w1;
  const float* w1_side;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* mu_a;
  const float* sigma_a;
  const float* mu_b;
  const float* sigma_b;
  const float* w_a;
  const float* w_b;
  void* workspace;
  int64_t workspace_bytes;
} tr_controller_weights;

/* Bytes of the optional controller workspace for model width d (a multiple of 64, 64 .. 16384;
 * -1 otherwise): 4 * 8 * ceil(d / 256) * 32 * 129.  Host only; no device call. */
int64_t tr_controller_workspace_bytes(int32_t d);

/* Pack the controller's first-layer weights (bf16 [128][d], out x in, row-major, device) into
 * the operand order tr_controller_route reads: w1_packed (bf16, d * 128 values, device, caller
 * owned, not overlapping w1) at [s][n][16] holds, for k-step s = 4 g + j and trunk unit n, the
 * channels 64 g + 8 j .. + 7 and 64 g + 32 + 8 j .. + 7 of row n.  d: a multiple of 64. */
tr_status tr_controller_pack_w1(const void* w1, void* w1_packed, int32_t d, void* stream);

/* Routing decisions at inference (the inference paragraph after Algorithm 1: the routers take
 * the hard argmax) for n_tokens tokens of one layer, written straight into the layouts the
 * attention calls read:
 *   x:    bf16 [n_tokens, d] residual states (e.g. [batch, T] flattened)
 *   side: float [n_tokens, d_side] side features psi_t (NULL if d_side = 0)
 *   mode: uint8 [n_tokens, heads]  argmax of each head's 3 logits (TR_MODE_*)
 *   bits: uint8 [n_tokens]         (2, 4, 8, 16)[argmax of the 4 width logits]
 * Ties go to the lowest index.  The trunk's first layer runs on the matrix cores with the bf16
 * x and w1 as exact operands and fp32 accumulation; everything after it is fp32 (the order of
 * the fp32 sums differs between the one- and two-launch forms).  n_tokens = 0 is a no-op.
 * TR_ERR_INVALID_ARG for a workspace smaller than tr_controller_workspace_bytes(d) or not
 * 16-byte aligned. */
tr_status tr_controller_route(const tr_controller_weights* w, const void* x, const float* side,
                              int64_t n_tokens, uint8_t* mode, uint8_t* bits, void* stream);

/* Expert FFN with a null expert (review page, "core formulas" item 3, Eq. (3)):
 *   FFN_t = sum_{j in S_t} p_tj / sum_{j' in S_t} p_tj' * f_j(RMSNorm(x_t)),  p_t = softmax(z_t),
 * over E experts plus the null expert f_0 = 0 (gate index 0), S_t the top_k largest p_t (ties to
 * the lower index), each expert a SwiGLU FFN f(u) = W2 (silu(W1 u) * (W3 u)) with no biases.
 * Products run on the matrix cores with fp32 accumulation: the gate and up products on bf16 x and
 * W1, W3 exactly (the RMSNorm scale applied to the fp32 sums); the down product on fp16 operands,
 * W2 rounded to fp16 once (exact for bf16 weights of magnitude 2^-14 .. 65504) and the hidden
 * activation rounded to fp16 (11 significant bits).  A weight of W2 or a hidden value beyond fp16's
 * range (|v| > 65504) sets the sticky TR_ERR_RANGE flag (tr_moe_status) and leaves the output
 * unspecified.  The gate logits come from the caller (e.g. an expert head of the controller,
 * Eq. (5)).  A handle owns the packed weights and the scratch of calls up to
 * max_tokens tokens. */
typedef struct {
  int32_t d;                /* model width: a multiple of 128, 128 .. 16384 */
  int32_t d_expert;         /* expert hidden width: a multiple of 128 */
  int32_t experts;          /* E: 1 .. 64 (the gate has E + 1 logits) */
  int32_t top_k;            /* 1 or 2 (1 with the null expert chosen = the MoD-style FFN skip) */
  int32_t max_tokens;       /* tokens per call, >= 1 */
} tr_moe_desc;

typedef struct tr_moe tr_moe;

/* Allocate a handle (device memory via hipMalloc on the current device); nothing on error. */
tr_status tr_moe_alloc(const tr_moe_desc* desc, tr_moe** out);

/* Free the handle's device memory (synchronizes the device).  NULL is a no-op. */
tr_status tr_moe_free(tr_moe* moe);

/* Copy the experts' weights into the handle, packed into the matrix-core operand order:
 *   w_gate, w_up: bf16 [E][d_expert][d]  (W1, W3: out x in, row-major)
 *   w_down:       bf16 [E][d][d_expert]  (W2: out x in)
 * Device pointers; asynchronous on `stream`, the inputs may be freed once the stream has
 * reached the call. */
tr_status tr_moe_set_weights(tr_moe* moe, const void* w_gate, const void* w_up, const void* w_down, void* stream);

/* Eq. (3) for n_tokens tokens (0 <= n_tokens <= max_tokens; 0 is a no-op):
 *   x:           bf16 [n_tokens, d] FFN inputs before Norm
 *   gate_logits: float [n_tokens, E + 1], index 0 = the null expert
 *   y:           float [n_tokens, d] receives FFN_t (a token whose choices are all the null
 *                expert gets zeros).  Deterministic: no atomics. */
tr_status tr_moe_ffn(tr_moe* moe, const void* x, const float* gate_logits, int32_t n_tokens, float* y, void* stream);

/* Sticky device flags of the handle, after synchronizing `stream`: TR_ERR_RANGE if a set_weights
 * or ffn call met a value outside fp16's range (see above), else TR_OK.  The flags persist for the
 * handle's lifetime. */
tr_status tr_moe_status(tr_moe* moe, void* stream);

/* Static description of a status code (never NULL). */
const char* tr_status_str(tr_status status);

#ifdef __cplusplus
}
#endif

#endif /* TRIROUTE_H_ */
