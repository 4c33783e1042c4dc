/*
 * sinkattn.h -- C ABI of the MI355X (gfx950) sink-attention library
 * (libsinkattn.so): grouped-query attention whose softmax carries one learned
 * logit per query head, for causal prefill and for split-KV decode.
 *
 * The operation.  "GPT-OSS on day 0" (Perplexity blog), section "Attention:
 * GQA with attention sinks": each attention head owns a trained sink
 * parameter that enters its softmax.  Section "Kernels for GPT-OSS /
 * Sink-Attention": the sink is an extra bias term of the softmax next to the
 * Q.K products; the softmax is computed online with the running maximum
 * subtracted; the running maximum is seeded with the head's sink and the
 * running scale with 1; and when the key range is split into chunks, only the
 * first chunk carries the sink.  In formula form, for query row q of head h
 * in GQA group g = h / (Hq/Hkv), over its visible keys J:
 *
 *     x_j = scale * q . k_j,   Z = exp(s_h) + sum_j exp(x_j),
 *     o   = sum_j exp(x_j) / Z * v_j          (the sink has no value row)
 *     lse = ln Z
 *
 * "Hosting Qwen on Blackwell" (Perplexity blog), section "Deployment on GB200
 * NVL72": KV caches are stored in HND order, heads leading and the tokens of
 * a head contiguous.  Every K/V argument below takes explicit strides, so HND
 * (token stride D, head stride T*D) is the natural layout; d must always be
 * the unit-stride dimension.
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers.  bf16 tensors are passed as void* holding
 *    IEEE bfloat16; sinks and partial states are fp32; lengths are int32.
 *  - Strides are in ELEMENTS, must be multiples of 8 (16 bytes) and >= 0;
 *    every bf16 pointer must be 16-byte aligned, fp32 pointers 4-byte aligned.
 *  - The caller allocates and owns every buffer.  The library allocates
 *    nothing, never synchronises, and enqueues all work on `stream` (a
 *    hipStream_t; NULL is the null stream), so calls can be graph-captured.
 *  - head_dim must be 64 or 128.  num_q_heads must be a multiple of
 *    num_kv_heads; query head h uses KV head h / (num_q_heads/num_kv_heads).
 *  - sinks[h] must be finite or -inf (-inf gives plain attention); +inf and
 *    NaN are undefined.  Device-resident lengths are not checked (see each
 *    function's preconditions); violating them is undefined behaviour.
 *  - Return codes: SINK_ATTN_OK (0), SINK_ATTN_EINVAL (-1, bad argument,
 *    nothing enqueued), SINK_ATTN_EUNSUPPORTED (-2, valid but not
 *    implemented, nothing enqueued), SINK_ATTN_ELAUNCH (-3, the HIP launch
 *    failed).  Every non-zero return sets a thread-local message readable
 *    through sink_attn_last_error().  All argument checks run on the host
 *    before any HIP call; no C++ exception crosses this boundary.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINK_ATTN_OK 0
#define SINK_ATTN_EINVAL (-1)
#define SINK_ATTN_EUNSUPPORTED (-2)
#define SINK_ATTN_ELAUNCH (-3)

/*
 * Prefill over packed variable-length sequences ("Hosting Qwen on
 * Blackwell", section "Prefillers": thousands of tokens of one request are
 * processed at once, so prefill is compute-bound; "GPT-OSS on day 0",
 * section "Kernels for GPT-OSS / Sink-Attention": the same sink-aware
 * attention serves prefill and decode).
 *
 *   q   [T, Hq, D] bf16: token t, head h at q + t*q_stride_tok + h*q_stride_head.
 *   k,v bf16: token t of KV head g at k + t*k_stride_tok + g*k_stride_head
 *       (HND [Hkv, T, D]: k_stride_tok = D, k_stride_head = T*D).
 *   sinks [Hq] fp32.
 *   cu_seqlens [num_seqs + 1] int32, device: sequence s owns packed tokens
 *       cu_seqlens[s] .. cu_seqlens[s+1]-1.  Precondition: cu_seqlens[0] = 0,
 *       non-decreasing, every length <= max_seqlen.  One sequence's keys are
 *       addressed with 32-bit byte offsets: max_seqlen * k_stride_tok * 2
 *       (and the same for v) must stay below 2^31, else SINK_ATTN_EUNSUPPORTED.
 *   max_seqlen: host-side upper bound of the sequence lengths (sizes the grid).
 *   scale: softmax scale applied to q.k (1/sqrt(D) is usual); the sink is
 *       not scaled.
 *   causal: 1 = key j visible to query i iff j <= i (positions inside the
 *       sequence); 0 = the whole sequence is visible.
 *   o [T, Hq, D] bf16 (output, round-to-nearest-even) with its own strides.
 *   lse: NULL, or fp32 [T, Hq] contiguous (output): ln Z of each row,
 *       natural-log units, sink included.
 * num_seqs = 0 or max_seqlen = 0 is a no-op.  o must not alias q, k or v.
 */
int sink_attn_prefill(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                      const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                      const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                      const float* sinks, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, float scale, int32_t causal,
                      void* o, int64_t o_stride_tok, int64_t o_stride_head,
                      float* lse, void* stream);

/*
 * Chunked prefill: per sequence a chunk of len_q new query tokens against
 * len_k >= len_q keys that hold the sequence's earlier tokens followed by the
 * chunk's own ("Hosting Qwen on Blackwell", section "Prefillers", prefills
 * long inputs on dedicated nodes; cutting an input into chunks over a cached
 * prefix is the plain extension).  Query i of the chunk sits at position
 * len_k - len_q + i of its sequence; causal = 1 lets it see keys
 * 0 .. len_k - len_q + i, causal = 0 all len_k keys.  cu_seqlens_q ==
 * cu_seqlens_k is exactly sink_attn_prefill.
 *   q, o [Tq, Hq, D] packed by cu_seqlens_q; k, v packed by cu_seqlens_k
 *       (token t of KV head g at k + t*k_stride_tok + g*k_stride_head).
 *   cu_seqlens_q, cu_seqlens_k [num_seqs + 1] int32, device.  Precondition:
 *       both start at 0 and are non-decreasing, every chunk length is at most
 *       max_seqlen_q and at most its sequence's key count; a sequence that
 *       breaks the last condition is skipped (its outputs are left unwritten).
 *       Each sequence's key count times k_stride_tok * 2 (and v's) must stay
 *       below 2^31 bytes (32-bit offsets; unchecked device values).
 *   lse: NULL, or fp32 [Tq, Hq] contiguous.
 *   Other arguments and errors as sink_attn_prefill.
 */
int sink_attn_prefill_chunked(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                              const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                              const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                              const float* sinks, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs,
                              int32_t max_seqlen_q, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, float scale, int32_t causal,
                              void* o, int64_t o_stride_tok, int64_t o_stride_head,
                              float* lse, void* stream);

/*
 * First half of split-KV decode: one query token per request against its
 * cached keys, with each request's key range cut into num_splits chunks of
 * split_size tokens ("GPT-OSS on day 0", section "Kernels for GPT-OSS /
 * Sink-Attention": attention is parallelised over heads and over the KV
 * length, and only the first chunk carries the sink; "Hosting Qwen on
 * Blackwell", section "Decoders": decode is memory-bound).
 *
 *   q [B, Hq, D] bf16: request b, head h at q + b*q_stride_b + h*q_stride_head.
 *   k_cache, v_cache bf16, HND per request: token j of KV head g of request
 *       b at base + b*kv_stride_b + g*kv_stride_head + j*kv_stride_tok (the
 *       two caches share the strides).
 *   seq_lens [B] int32, device.  Precondition: 0 <= seq_lens[b] <= max_ctx.
 *   split_size: tokens per chunk, a positive multiple of 64, with
 *       split_size * kv_stride_tok * 2 < 2^31 (else SINK_ATTN_EUNSUPPORTED).
 *   num_splits: chunks per request; num_splits * split_size >= max_ctx.
 *   Outputs, for row (b, h) and chunk c = 0 .. num_splits-1, chunk c covering
 *   tokens [c*split_size, min((c+1)*split_size, seq_lens[b])):
 *     part_o [B, Hq, num_splits, D] fp32: the chunk's output, already divided
 *         by its own denominator;
 *     part_m [B, Hq, num_splits] fp32: the chunk's running maximum (natural-
 *         log units; chunk 0 includes the sink);
 *     part_d [B, Hq, num_splits] fp32: the chunk's denominator relative to
 *         exp(part_m) (chunk 0 includes the sink term).
 *   An empty chunk without the sink is written as (o, m, d) = (0, -inf, 0).
 * Feed the partials to sink_attn_merge_states on the same stream.
 */
int sink_attn_decode_split(const void* q, int64_t q_stride_b, int64_t q_stride_head,
                           const void* k_cache, const void* v_cache, int64_t kv_stride_b,
                           int64_t kv_stride_head, int64_t kv_stride_tok,
                           const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                           const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float scale, int32_t split_size,
                           int32_t num_splits, float* part_o, float* part_m,
                           float* part_d, void* stream);

/*
 * Multi-token decode, split over the KV length: the speculative and MTP
 * decoders of "GPT-OSS on day 0" (section "Internal inference engine") and
 * "Hosting Qwen on Blackwell" (section "Decoders") verify q_len new tokens
 * per request in one pass.  The new tokens are already the last q_len of
 * the request's cache; new token t (0 <= t < q_len) of request b attends, as
 * in sink_attn_decode_split, to cached tokens 0 .. seq_lens[b] - q_len + t
 * (causal among the new tokens).  A row that sees no token sees only the
 * sink.  q_len = 1 is exactly sink_attn_decode_split.
 *   q [B, q_len, Hq, D] bf16: new token t of request b, head h at
 *     q + b*q_stride_b + t*q_stride_tok + h*q_stride_head (d unit-stride).
 *   caches, seq_lens, sinks, scale, split_size, num_splits: as in
 *     sink_attn_decode_split.
 *   part_o [B, q_len, Hq, num_splits, D], part_m / part_d
 *     [B, q_len, Hq, num_splits] fp32 contiguous (caller-allocated, outputs),
 *     the same per-chunk states; merge them with sink_attn_merge_states with
 *     batch = B * q_len (output row (b, t, h) is row (b*q_len + t, h)).
 * The kernel is meant for small q_len (one workgroup serves 16 (token, head)
 * columns of a GQA group); any q_len >= 1 is accepted.
 * Errors: as sink_attn_decode_split, plus SINK_ATTN_EINVAL for q_len < 1 or a
 * q_stride_tok that is negative or not a multiple of 8.
 */
int sink_attn_decode_multi_split(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                 int64_t q_stride_head, int32_t q_len,
                                 const void* k_cache, const void* v_cache, int64_t kv_stride_b,
                                 int64_t kv_stride_head, int64_t kv_stride_tok,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                                 const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float scale, int32_t split_size,
                                 int32_t num_splits, float* part_o, float* part_m,
                                 float* part_d, void* stream);

/*
 * A chunk size for the split-KV decode calls above and below, chosen from the
 * launch shape ("GPT-OSS on day 0", section "Kernels for GPT-OSS /
 * Sink-Attention": decode is parallelised over the KV length as well as over
 * heads; the best cut depends on the shape).  The request lengths of a
 * decode are device values; a caller that also holds them on the host passes
 * them in seq_lens_host, else NULL.
 *  - Lengths given and (nearly) equal (their mean >= 0.9 x their longest):
 *    the longest of 8192, 4096, 2048, 1024 tokens that is needed to cover the
 *    longest request and still gives every fourth SIMD of the current device
 *    a (request, KV head, column slice, chunk) unit -- long chunks write fewer
 *    chunk states for the merge, and equal units finish together.  When even
 *    1024 leaves fewer units than that (a few requests), the shortest multiple
 *    of 128 tokens that gives at most one unit per CU.
 *  - Otherwise (ragged or unknown lengths): 1024, or 2048 when chunks of 2048
 *    at max_ctx still give every SIMD four units -- short chunks keep a
 *    ragged batch's longest requests from finishing alone.
 * Always a positive multiple of 64.  Size the partials with num_splits =
 * ceil(max_ctx / split).
 *   batch, max_ctx >= 0; q_len >= 1; heads and head_dim as for
 *   sink_attn_decode_multi_split; seq_lens_host: NULL or batch host int32
 *   lengths, each in [0, max_ctx].
 * Returns the split size, or SINK_ATTN_EINVAL / SINK_ATTN_EUNSUPPORTED (with a
 * message) for invalid arguments.  Enqueues nothing, reads no device memory.
 */
int32_t sink_attn_decode_split_size(int32_t batch, int32_t max_ctx, int32_t q_len,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    const int32_t* seq_lens_host);

/*
 * Second half of split-KV decode: merge each row's chunk states by their
 * log-sum-exp weights (the pages state that chunks are formed and that only
 * the first carries the sink; the merge is the exact recombination this
 * implies):  M = max_c m_c,  w_c = d_c * exp(m_c - M),
 *            o = sum_c w_c o_c / sum_c w_c,  lse = M + ln sum_c w_c.
 * Chunks with m_c = -inf get weight 0; a row with no weight gives o = 0 and
 * lse = -inf.
 *   part_o, part_m, part_d: as written by sink_attn_decode_split (or by
 *     sink_attn_decode_multi_split, with batch = B * q_len).
 *   o [B, Hq, D] bf16 (output): row (b, h) at o + b*o_stride_b + h*o_stride_head.
 *   lse: NULL, or fp32 [B, Hq] contiguous (output).
 */
int sink_attn_merge_states(const float* part_o, const float* part_m, const float* part_d,
                           int32_t batch, int32_t num_q_heads, int32_t num_splits,
                           int32_t head_dim, void* o, int64_t o_stride_b,
                           int64_t o_stride_head, float* lse, void* stream);

/*
 * Append new tokens' K and V to per-request HND caches, the step between
 * prefill (or a decode step) and the decode that streams the caches
 * ("Hosting Qwen on Blackwell": section "Deployment on GB200 NVL72" keeps
 * caches in HND order; sections "Prefillers" / "Decoders": prefill fills the
 * caches the decoders read).  A pure copy, bit-exact:
 *   for request b, new token t < cu_seqlens_new[b+1] - cu_seqlens_new[b],
 *   KV head g:  cache[b, g, cache_pos[b] + t, :] = new[cu_seqlens_new[b] + t, g, :]
 *   k_new, v_new bf16: token t of KV head g at k_new + t*new_stride_tok +
 *       g*new_stride_head (token-major [T, Hkv, D]: stride_tok = Hkv*D,
 *       stride_head = D); d unit-stride.
 *   cu_seqlens_new [num_seqs + 1] int32, device; cache_pos [num_seqs] int32,
 *       device (first slot written for each request).
 *   k_cache, v_cache bf16 (in/out): element (b, g, slot j, d) at
 *       b*kv_stride_b + g*kv_stride_head + j*kv_stride_tok + d.
 *   max_new: host-side bound of the new-token counts (sizes the grid).
 * Slots outside [0, max_ctx) are not written (the tokens that would land there
 * are dropped); every other cache slot is left unchanged.  The new rows must
 * not overlap the caches.  num_seqs, max_new or max_ctx = 0 is a no-op.
 * Errors: as the other calls (null pointers, 16-byte alignment, strides,
 * head_dim 64 / 128).
 */
int sink_attn_kv_append(const void* k_new, const void* v_new, int64_t new_stride_tok,
                        int64_t new_stride_head, const int32_t* cu_seqlens_new,
                        const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                        void* k_cache, void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                        int64_t kv_stride_tok, int32_t max_ctx, int32_t num_kv_heads,
                        int32_t head_dim, void* stream);

/*
 * Split decode and merge in one launch: the work of
 * sink_attn_decode_multi_split (bf16 caches, or FP8 E4M3 caches when k_scale
 * and v_scale are given -- both or neither) followed by
 * sink_attn_merge_states, with the merge done by whichever workgroup
 * finishes the last chunk of a (request, KV head, column slice): it counts
 * itself in on `counters`, and the last arrival merges that slice's rows.
 * Same results as the two calls (the merge is the same code; chunks past a
 * request's end hold (0, -inf, 0) and add nothing, so they are left out).
 *   part_o, part_m, part_d: as sink_attn_decode_multi_split, except that the
 *       states of chunks past a request's end (chunk c > 0 with
 *       c * split_size >= seq_lens[b]) are not written.
 *   counters: int32, device, at least batch * num_kv_heads *
 *       ceil(q_len * (num_q_heads / num_kv_heads) / 16) elements, all zero
 *       before the first call; every call leaves them zero.  Calls that run
 *       concurrently must not share counters.
 *   o [B, q_len, Hq, D] bf16: new token t of request b, head h at
 *       o + b*o_stride_b + t*o_stride_tok + h*o_stride_head (d unit-stride).
 *   lse: NULL, or fp32 [B, q_len, Hq] contiguous.
 *   Other arguments and errors as sink_attn_decode_multi_split.
 */
int sink_attn_decode_fused(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                           int64_t q_stride_head, int32_t q_len, const void* k_cache,
                           const void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                           int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                           const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                           const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float scale, int32_t split_size, int32_t num_splits,
                           float* part_o, float* part_m, float* part_d, int32_t* counters,
                           void* o, int64_t o_stride_b, int64_t o_stride_tok,
                           int64_t o_stride_head, float* lse, void* stream);

/*
 * Split decode and merge for ragged batches, in two launches: as
 * sink_attn_decode_multi_split followed by sink_attn_merge_states, except
 * that chunks past a request's end (chunk index >= max(1, ceil(seq_lens[b] /
 * split_size))) write no state and the merge stops at each request's last
 * chunk with keys -- their state (0, -inf, 0) would add only exact zeros, so
 * o and lse are bitwise those of the two calls.  Writing those states is
 * what chunks past the end cost in a ragged batch ("Hosting Qwen on
 * Blackwell", section "Decoders": decode is bound by memory traffic).
 *   Arguments as sink_attn_decode_fused without counters: part_o / part_m /
 *   part_d [B, q_len, Hq, num_splits(, D)] fp32 caller-allocated scratch
 *   (entries of chunks past a request's end are left as they were); o
 *   [B, q_len, Hq, D] bf16 (output, 16-byte aligned, strides multiples of 8
 *   elements); lse NULL or fp32 [B, q_len, Hq] (output).  k_scale / v_scale:
 *   both NULL (bf16 caches) or both given (FP8 E4M3 codes, as
 *   sink_attn_decode_multi_split_fp8).
 * Errors: as sink_attn_decode_fused (no counters to check).
 */
int sink_attn_decode_merged(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                            int64_t q_stride_head, int32_t q_len, const void* k_cache,
                            const void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                            int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                            const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                            const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, float scale, int32_t split_size, int32_t num_splits,
                            float* part_o, float* part_m, float* part_d, void* o,
                            int64_t o_stride_b, int64_t o_stride_tok, int64_t o_stride_head,
                            float* lse, void* stream);

/*
 * sink_attn_decode_merged without the caller's partial buffers, for callers
 * that cannot allocate device memory around the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The chunk
 * states live in a device array the library holds on each GPU it runs on
 * (2^25 fp32 = 128 MiB, kept until the process ends); the call itself
 * allocates and frees nothing.
 *   Arguments, outputs and results as sink_attn_decode_merged (bitwise the
 *   same o and lse), minus part_o / part_m / part_d.
 *   Limit: batch * q_len * num_q_heads * num_splits * (head_dim + 2) <= 2^25,
 *   else SINK_ATTN_EINVAL (nothing enqueued).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (concurrent streams, threads) race and give undefined results; calls
 *   ordered on one stream are safe.  Nothing in the array needs to start at
 *   zero (every state the merge reads is written by the same call).  The
 *   array is found on the device current at the call (stream must belong to
 *   it); the first call on a device looks up its address
 *   (SINK_ATTN_ELAUNCH if that fails).
 */
int sink_attn_decode_merged_noalloc(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                    int64_t q_stride_head, int32_t q_len, const void* k_cache,
                                    const void* v_cache, int64_t kv_stride_b,
                                    int64_t kv_stride_head, int64_t kv_stride_tok,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                                    const float* sinks, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, float scale,
                                    int32_t split_size, int32_t num_splits, void* o,
                                    int64_t o_stride_b, int64_t o_stride_tok,
                                    int64_t o_stride_head, float* lse, void* stream);

/*
 * FP8 KV cache.  The pages speak of FP8 only for weights; decode, though, is
 * bound by the bytes of the cache it streams ("Hosting Qwen on Blackwell",
 * section "Decoders"), and one byte per element halves them.  Format: OCP FP8
 * E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite value 448), one byte per
 * element, in the same HND layout as the bf16 caches, with one fp32
 * dequantization scale per KV head: the cached value of KV head g is
 * e4m3(code) * k_scale[g] (v_scale[g] for V).
 *
 * sink_attn_decode_multi_split_fp8: sink_attn_decode_multi_split over FP8
 * caches -- the same chunk states (part_o, part_m, part_d, same shapes and
 * meaning), computed on the dequantized cache.  Strides are in elements
 * (= bytes) and must be multiples of 16; k_scale, v_scale [num_kv_heads]
 * fp32, device, both required.  q_len = 1 is plain split decode.  Feed the
 * partials to sink_attn_merge_states.  Errors: as
 * sink_attn_decode_multi_split.
 */
int sink_attn_decode_multi_split_fp8(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                     int64_t q_stride_head, int32_t q_len, const void* k_cache,
                                     const void* v_cache, int64_t kv_stride_b,
                                     int64_t kv_stride_head, int64_t kv_stride_tok,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                                     const float* sinks, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, float scale,
                                     int32_t split_size, int32_t num_splits, float* part_o,
                                     float* part_m, float* part_d, void* stream);

/*
 * sink_attn_kv_append_fp8: sink_attn_kv_append into FP8 caches.  The new rows
 * are bf16 as for sink_attn_kv_append; element x of KV head g is stored as the
 * E4M3 code of fp32(x) * fp32(1 / k_scale[g]) (v_scale[g] for V): the
 * reciprocal correctly rounded to fp32, the product rounded to fp32, then
 * rounded to nearest (ties to even) and saturated to +-448; a NaN gives a NaN
 * code.  Cache strides in elements (= bytes), multiples of 8.  Errors: as
 * sink_attn_kv_append, plus SINK_ATTN_EINVAL for a missing scale.
 */
int sink_attn_kv_append_fp8(const void* k_new, const void* v_new, int64_t new_stride_tok,
                            int64_t new_stride_head, const int32_t* cu_seqlens_new,
                            const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                            void* k_cache, void* v_cache, int64_t kv_stride_b,
                            int64_t kv_stride_head, int64_t kv_stride_tok, const float* k_scale,
                            const float* v_scale, int32_t max_ctx, int32_t num_kv_heads,
                            int32_t head_dim, void* stream);

/*
 * Paged (block-table) KV cache.  The pages keep each request's cache in HND
 * order ("Hosting Qwen on Blackwell", section "Deployment on GB200 NVL72");
 * a serving engine holds it in fixed-size pages instead of one contiguous
 * slab per request (not on the pages; reading: HND inside each page).
 *   k_pages, v_pages: [num_pages, Hkv, page_size, D], bf16 -- or FP8 E4M3
 *       codes when k_scale and v_scale are given (both or neither) -- with
 *       element strides page_stride, kv_stride_head, kv_stride_tok (d
 *       unit-stride; multiples of 8 bf16 / 16 FP8 elements).
 *   page_size: tokens per page, a power of two in [16, 2^20].
 *   block_tables [batch, pages_per_seq] int32, device, row stride bt_stride:
 *       request b's token j lives in page block_tables[b*bt_stride +
 *       j / page_size], row j % page_size.  Precondition: every entry a
 *       request's length reaches is a valid page index, and seq_lens[b] <=
 *       pages_per_seq * page_size (unchecked device values).
 * sink_attn_decode_paged_split: sink_attn_decode_multi_split (or its FP8
 * form) over such pages -- the same chunk states, same shapes; max_ctx is
 * pages_per_seq * page_size.  Chunks may span at most 255 pages
 * (split_size <= 254 * page_size, else SINK_ATTN_EUNSUPPORTED).
 */
int sink_attn_decode_paged_split(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                 int64_t q_stride_head, int32_t q_len, const void* k_pages,
                                 const void* v_pages, int64_t page_stride, int64_t kv_stride_head,
                                 int64_t kv_stride_tok, int32_t page_size,
                                 const int32_t* block_tables, int64_t bt_stride,
                                 int32_t pages_per_seq, const float* k_scale, const float* v_scale,
                                 const int32_t* seq_lens, int32_t batch, const float* sinks,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 float scale, int32_t split_size, int32_t num_splits,
                                 float* part_o, float* part_m, float* part_d, void* stream);

/*
 * sink_attn_kv_append_paged: sink_attn_kv_append (a copy into bf16 pages) or
 * sink_attn_kv_append_fp8 (quantizing into FP8 pages, when the scales are
 * given) through a block table: new token t of request b goes to logical slot
 * cache_pos[b] + t, i.e. page block_tables[b*bt_stride + slot / page_size],
 * row slot % page_size; slots at or past pages_per_seq * page_size are
 * dropped.  Layout, strides and preconditions as for
 * sink_attn_decode_paged_split.
 */
int sink_attn_kv_append_paged(const void* k_new, const void* v_new, int64_t new_stride_tok,
                              int64_t new_stride_head, const int32_t* cu_seqlens_new,
                              const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                              void* k_pages, void* v_pages, int64_t page_stride,
                              int64_t kv_stride_head, int64_t kv_stride_tok, int32_t page_size,
                              const int32_t* block_tables, int64_t bt_stride,
                              int32_t pages_per_seq, const float* k_scale, const float* v_scale,
                              int32_t num_kv_heads, int32_t head_dim, void* stream);

/* Message of the last failed call on this thread ("" if none).  The pointer
 * stays valid until the next call into the library on the same thread. */
const char* sink_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */
