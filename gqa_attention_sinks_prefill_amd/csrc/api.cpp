// C ABI of libsinkattn.so: argument validation (host only, before any HIP
// call), launch-shape selection, and error reporting.  The operations and
// their layouts are documented in include/sinkattn.h.
#include "sinkattn.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
bool stride_ok(int64_t s) { return s >= 0 && s % 8 == 0; }

int check_heads(int32_t hq, int32_t hkv, int32_t d) {
  if (hq <= 0 || hkv <= 0) return fail(SINK_ATTN_EINVAL, "head counts must be positive (Hq=%d, Hkv=%d)", hq, hkv);
  if (hq % hkv != 0) return fail(SINK_ATTN_EINVAL, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", hq, hkv);
  if (d != 64 && d != 128) return fail(SINK_ATTN_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", d);
  return SINK_ATTN_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SINK_ATTN_EINVAL, "scale must be finite and positive");
  return SINK_ATTN_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SINK_ATTN_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return SINK_ATTN_OK;
}

}  // namespace

extern "C" {

const char* sink_attn_last_error(void) { return g_err; }

int sink_attn_prefill_chunked(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                              const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                              const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                              const float* sinks, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs,
                              int32_t max_seqlen_q, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, float scale, int32_t causal,
                              void* o, int64_t o_stride_tok, int64_t o_stride_head,
                              float* lse, void* stream) {
  const int32_t* cu_seqlens = cu_seqlens_q;
  const int32_t max_seqlen = max_seqlen_q;
  g_err[0] = '\0';
  if (num_seqs < 0 || max_seqlen < 0) return fail(SINK_ATTN_EINVAL, "num_seqs and max_seqlen must be >= 0");
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  if (int rc = check_scale(scale)) return rc;
  if (causal != 0 && causal != 1) return fail(SINK_ATTN_EINVAL, "causal must be 0 or 1");
  if (num_seqs == 0 || max_seqlen == 0) return SINK_ATTN_OK;
  if (!q || !k || !v || !sinks || !cu_seqlens || !cu_seqlens_k || !o)
    return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(SINK_ATTN_EINVAL, "q, k, v and o must be 16-byte aligned");
  if (!aligned(sinks, 4) || !aligned(cu_seqlens, 4) || !aligned(cu_seqlens_k, 4) ||
      (lse && !aligned(lse, 4)))
    return fail(SINK_ATTN_EINVAL, "sinks, cu_seqlens and lse must be 4-byte aligned");
  if (!stride_ok(q_stride_tok) || !stride_ok(q_stride_head) || !stride_ok(k_stride_tok) ||
      !stride_ok(k_stride_head) || !stride_ok(v_stride_tok) || !stride_ok(v_stride_head) ||
      !stride_ok(o_stride_tok) || !stride_ok(o_stride_head))
    return fail(SINK_ATTN_EINVAL, "strides must be non-negative multiples of 8 elements");
  // one sequence's keys are addressed with 32-bit byte offsets (the key count
  // of a chunked call is on the device; its bound is a documented precondition)
  if (cu_seqlens_k == cu_seqlens_q &&
      static_cast<int64_t>(max_seqlen) * (k_stride_tok > v_stride_tok ? k_stride_tok : v_stride_tok) * 2 >
          0x7fffffffLL)
    return fail(SINK_ATTN_EUNSUPPORTED, "max_seqlen * token stride spans more than 2 GiB");

  const int group = num_q_heads / num_kv_heads;
  const int hpw = sinkattn::prefill_heads_per_workgroup(group);
  const int rows = sinkattn::prefill_rows_per_workgroup(group, head_dim);
  const int64_t n_qtiles = (max_seqlen + rows - 1) / rows;
  const int64_t num_blocks = n_qtiles * num_seqs * (num_q_heads / hpw);
  if (num_blocks > 0x7fffffff) return fail(SINK_ATTN_EUNSUPPORTED, "problem too large for one launch");

  sinkattn::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.k = static_cast<const uint16_t*>(k);
  a.k_st = k_stride_tok;
  a.k_sh = k_stride_head;
  a.v = static_cast<const uint16_t*>(v);
  a.v_st = v_stride_tok;
  a.v_sh = v_stride_head;
  a.sinks = sinks;
  a.cu_seqlens = cu_seqlens;
  a.cu_seqlens_k = cu_seqlens_k;
  a.o = static_cast<uint16_t*>(o);
  a.o_st = o_stride_tok;
  a.o_sh = o_stride_head;
  a.lse = lse;
  a.num_seqs = num_seqs;
  a.n_qtiles = static_cast<int32_t>(n_qtiles);
  a.num_q_heads = num_q_heads;
  a.group = group;
  a.head_groups = num_q_heads / hpw;
  a.causal = causal;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launched(sinkattn::launch_prefill(a, head_dim, num_blocks, static_cast<hipStream_t>(stream)),
                  "prefill");
}

int sink_attn_prefill(const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                      const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                      const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                      const float* sinks, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, float scale, int32_t causal,
                      void* o, int64_t o_stride_tok, int64_t o_stride_head,
                      float* lse, void* stream) {
  // every sequence's queries are all of its tokens: the chunked form with
  // one boundary table for both
  return sink_attn_prefill_chunked(q, q_stride_tok, q_stride_head, k, k_stride_tok, k_stride_head,
                                   v, v_stride_tok, v_stride_head, sinks, cu_seqlens, cu_seqlens,
                                   num_seqs, max_seqlen, num_q_heads, num_kv_heads, head_dim,
                                   scale, causal, o, o_stride_tok, o_stride_head, lse, stream);
}

// Multi-token split decode over bf16 caches (k_scale == nullptr) or FP8 E4M3
// caches with per-KV-head scales; per-request caches, or pages through a block
// table (block_tables != nullptr: kv_stride_b is then the page stride).
static int decode_multi_split(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                              int64_t q_stride_head, int32_t q_len, const void* k_cache,
                              const void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                              int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int64_t bt_stride, int32_t page_size,
                              const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                              const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, float scale, int32_t split_size, int32_t num_splits,
                              float* part_o, float* part_m, float* part_d, void* stream,
                              int32_t* counters = nullptr, void* o = nullptr, int64_t o_stride_b = 0,
                              int64_t o_stride_tok = 0, int64_t o_stride_head = 0,
                              float* lse = nullptr, bool merged = false,
                              bool use_scratch = false) {
  const bool fp8 = k_scale != nullptr || v_scale != nullptr;
  const bool fused = counters != nullptr || o != nullptr;
  const bool paged = page_size != 0;
  const int64_t elem = fp8 ? 1 : 2;           // bytes per cached element
  if (batch < 0 || max_ctx < 0) return fail(SINK_ATTN_EINVAL, "batch and max_ctx must be >= 0");
  int page_shift = 0;
  if (paged) {
    if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
      return fail(SINK_ATTN_EINVAL, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
    while ((1 << page_shift) < page_size) ++page_shift;
    if (bt_stride < 0) return fail(SINK_ATTN_EINVAL, "block_tables row stride must be >= 0");
  }
  if (q_len < 1) return fail(SINK_ATTN_EINVAL, "q_len must be >= 1 (got %d)", q_len);
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  if (int rc = check_scale(scale)) return rc;
  if (split_size <= 0 || split_size % 64 != 0)
    return fail(SINK_ATTN_EINVAL, "split_size must be a positive multiple of 64 (got %d)", split_size);
  if (num_splits <= 0) return fail(SINK_ATTN_EINVAL, "num_splits must be positive");
  if (static_cast<int64_t>(num_splits) * split_size < max_ctx)
    return fail(SINK_ATTN_EINVAL, "num_splits * split_size (%lld) does not cover max_ctx (%d)",
                static_cast<long long>(num_splits) * split_size, max_ctx);
  // a chunk spans at most split/page + 1 pages; the kernel holds 256 entries
  if (paged && (split_size + page_size - 1) / page_size + 1 > 256)
    return fail(SINK_ATTN_EUNSUPPORTED, "split_size %d spans more than 255 pages of %d tokens",
                split_size, page_size);
  if (batch == 0) return SINK_ATTN_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !sinks ||
      (!use_scratch && (!part_o || !part_m || !part_d)) || (paged && !block_tables))
    return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  if (paged && !aligned(block_tables, 4))
    return fail(SINK_ATTN_EINVAL, "block_tables must be 4-byte aligned");
  if (fused) {
    if ((!merged && !counters) || !o) return fail(SINK_ATTN_EINVAL, "a required pointer is null");
    if ((!merged && !aligned(counters, 4)) || !aligned(o, 16) || (lse && !aligned(lse, 4)))
      return fail(SINK_ATTN_EINVAL, "counters and lse must be 4-byte aligned, o 16-byte aligned");
    if (!stride_ok(o_stride_b) || !stride_ok(o_stride_tok) || !stride_ok(o_stride_head))
      return fail(SINK_ATTN_EINVAL, "output strides must be non-negative multiples of 8 elements");
  }
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given, 4-byte aligned");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(SINK_ATTN_EINVAL, "q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(seq_lens, 4) || !aligned(sinks, 4) || !aligned(part_o, 4) || !aligned(part_m, 4) ||
      !aligned(part_d, 4))   // (null when the scratch array holds them)
    return fail(SINK_ATTN_EINVAL, "seq_lens, sinks and the partial buffers must be 4-byte aligned");
  if (!stride_ok(q_stride_b) || !stride_ok(q_stride_tok) || !stride_ok(q_stride_head))
    return fail(SINK_ATTN_EINVAL, "query strides must be non-negative multiples of 8 elements");
  // cache rows start on 16 bytes: 8 bf16 or 16 FP8 elements
  const int64_t kv_mult = 16 / elem;
  for (int64_t st : {kv_stride_b, kv_stride_head, kv_stride_tok})
    if (st < 0 || st % kv_mult != 0)
      return fail(SINK_ATTN_EINVAL, "cache strides must be non-negative multiples of %lld elements",
                  static_cast<long long>(kv_mult));
  // a chunk (a 16-key block of a page) of one head is addressed with 32-bit offsets
  if (static_cast<int64_t>(paged ? 16 : split_size) * kv_stride_tok * elem > 0x7fffffffLL)
    return fail(SINK_ATTN_EUNSUPPORTED, "split_size * kv_stride_tok spans more than 2 GiB");

  const int group = num_q_heads / num_kv_heads;
  const int64_t ncols = static_cast<int64_t>(q_len) * group;
  if (ncols > 0x7fffffff) return fail(SINK_ATTN_EUNSUPPORTED, "problem too large for one launch");
  const int cols_per_block = 16 * sinkattn::decode_column_blocks(static_cast<int>(ncols), head_dim);
  const int64_t head_slices = (ncols + cols_per_block - 1) / cols_per_block;
  const int64_t num_blocks = static_cast<int64_t>(batch) * num_kv_heads * head_slices * num_splits;
  if (ncols > 0x7fffffff || num_blocks > 0x7fffffff)
    return fail(SINK_ATTN_EUNSUPPORTED, "problem too large for one launch");
  if (use_scratch) {
    // the chunk states live in the library's device scratch array
    const int64_t rows = static_cast<int64_t>(batch) * q_len * num_q_heads;
    const int64_t need = rows * num_splits * (head_dim + 2);
    if (need > sinkattn::kDecodeScratchFloats)
      return fail(SINK_ATTN_EINVAL,
                  "the chunk states need %lld fp32 (batch * q_len * num_q_heads * num_splits * "
                  "(head_dim + 2)); the scratch holds %lld",
                  static_cast<long long>(need), static_cast<long long>(sinkattn::kDecodeScratchFloats));
    float* base = nullptr;
    const hipError_t e = sinkattn::decode_scratch(&base);
    if (e != hipSuccess)
      return fail(SINK_ATTN_ELAUNCH, "device address of the scratch array: %s", hipGetErrorString(e));
    part_o = base;
    part_m = base + rows * num_splits * head_dim;
    part_d = part_m + rows * num_splits;
  }

  sinkattn::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_sb = q_stride_b;
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  a.kv_sb = paged ? 0 : kv_stride_b;
  a.kv_sh = kv_stride_head;
  a.kv_st = kv_stride_tok;
  a.block_tables = paged ? block_tables : nullptr;
  a.bt_stride = bt_stride;
  a.kv_sp = paged ? kv_stride_b : 0;
  a.page_shift = page_shift;
  a.seq_lens = seq_lens;
  a.sinks = sinks;
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_d = part_d;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.q_len = q_len;
  a.ncols = static_cast<int32_t>(ncols);
  a.head_slices = static_cast<int32_t>(head_slices);
  a.batch = batch;
  a.split_size = split_size;
  a.num_splits = num_splits;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.skip_empty = merged ? 1 : 0;
  if (fused) {
    a.counters = merged ? nullptr : counters;
    a.merge.part_o = part_o;
    a.merge.part_m = part_m;
    a.merge.part_d = part_d;
    a.merge.o = static_cast<uint16_t*>(o);
    a.merge.o_sb = o_stride_b;
    a.merge.o_st = o_stride_tok;
    a.merge.o_sh = o_stride_head;
    a.merge.lse = lse;
    a.merge.rows = static_cast<int32_t>(static_cast<int64_t>(batch) * q_len * num_q_heads);
    a.merge.q_len = q_len;
    a.merge.num_q_heads = num_q_heads;
    a.merge.num_splits = num_splits;
  }
  const int rc = launched(sinkattn::launch_decode_split(a, head_dim, num_blocks,
                                                        static_cast<hipStream_t>(stream)),
                          "decode_split");
  if (rc != SINK_ATTN_OK || !merged) return rc;
  a.merge.seq_lens = seq_lens;
  a.merge.split_size = split_size;
  return launched(sinkattn::launch_merge(a.merge, head_dim, static_cast<hipStream_t>(stream)),
                  "merge_states");
}

int sink_attn_decode_multi_split(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                 int64_t q_stride_head, int32_t q_len,
                                 const void* k_cache, const void* v_cache, int64_t kv_stride_b,
                                 int64_t kv_stride_head, int64_t kv_stride_tok,
                                 const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                                 const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float scale, int32_t split_size,
                                 int32_t num_splits, float* part_o, float* part_m,
                                 float* part_d, void* stream) {
  g_err[0] = '\0';
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_cache, v_cache,
                            kv_stride_b, kv_stride_head, kv_stride_tok, nullptr, nullptr, nullptr, 0,
                            0, seq_lens,
                            batch, max_ctx, sinks, num_q_heads, num_kv_heads, head_dim, scale,
                            split_size, num_splits, part_o, part_m, part_d, stream);
}

int sink_attn_decode_multi_split_fp8(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                     int64_t q_stride_head, int32_t q_len, const void* k_cache,
                                     const void* v_cache, int64_t kv_stride_b,
                                     int64_t kv_stride_head, int64_t kv_stride_tok,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                                     const float* sinks, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, float scale,
                                     int32_t split_size, int32_t num_splits, float* part_o,
                                     float* part_m, float* part_d, void* stream) {
  g_err[0] = '\0';
  if (!k_scale || !v_scale) return fail(SINK_ATTN_EINVAL, "k_scale and v_scale are required");
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_cache, v_cache,
                            kv_stride_b, kv_stride_head, kv_stride_tok, k_scale, v_scale, nullptr, 0,
                            0, seq_lens,
                            batch, max_ctx, sinks, num_q_heads, num_kv_heads, head_dim, scale,
                            split_size, num_splits, part_o, part_m, part_d, stream);
}

int sink_attn_decode_fused(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                           int64_t q_stride_head, int32_t q_len, const void* k_cache,
                           const void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                           int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                           const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                           const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float scale, int32_t split_size, int32_t num_splits,
                           float* part_o, float* part_m, float* part_d, int32_t* counters,
                           void* o, int64_t o_stride_b, int64_t o_stride_tok,
                           int64_t o_stride_head, float* lse, void* stream) {
  g_err[0] = '\0';
  if ((k_scale == nullptr) != (v_scale == nullptr))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given or both be null");
  if (batch > 0 && (!counters || !o)) return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_cache, v_cache,
                            kv_stride_b, kv_stride_head, kv_stride_tok, k_scale, v_scale, nullptr, 0,
                            0, seq_lens, batch, max_ctx, sinks, num_q_heads, num_kv_heads,
                            head_dim, scale, split_size, num_splits, part_o, part_m, part_d,
                            stream, counters, o, o_stride_b, o_stride_tok, o_stride_head, lse);
}

int sink_attn_decode_merged(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                            int64_t q_stride_head, int32_t q_len, const void* k_cache,
                            const void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                            int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                            const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                            const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, float scale, int32_t split_size, int32_t num_splits,
                            float* part_o, float* part_m, float* part_d, void* o,
                            int64_t o_stride_b, int64_t o_stride_tok, int64_t o_stride_head,
                            float* lse, void* stream) {
  g_err[0] = '\0';
  if ((k_scale == nullptr) != (v_scale == nullptr))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given or both be null");
  if (batch > 0 && !o) return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_cache, v_cache,
                            kv_stride_b, kv_stride_head, kv_stride_tok, k_scale, v_scale, nullptr, 0,
                            0, seq_lens, batch, max_ctx, sinks, num_q_heads, num_kv_heads,
                            head_dim, scale, split_size, num_splits, part_o, part_m, part_d,
                            stream, nullptr, o, o_stride_b, o_stride_tok, o_stride_head, lse, true);
}

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
                                    int64_t o_stride_head, float* lse, void* stream) {
  g_err[0] = '\0';
  if ((k_scale == nullptr) != (v_scale == nullptr))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given or both be null");
  if (batch > 0 && !o) return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_cache, v_cache,
                            kv_stride_b, kv_stride_head, kv_stride_tok, k_scale, v_scale, nullptr, 0,
                            0, seq_lens, batch, max_ctx, sinks, num_q_heads, num_kv_heads,
                            head_dim, scale, split_size, num_splits, nullptr, nullptr, nullptr,
                            stream, nullptr, o, o_stride_b, o_stride_tok, o_stride_head, lse, true,
                            true);
}

int sink_attn_decode_paged_split(const void* q, int64_t q_stride_b, int64_t q_stride_tok,
                                 int64_t q_stride_head, int32_t q_len, const void* k_pages,
                                 const void* v_pages, int64_t page_stride, int64_t kv_stride_head,
                                 int64_t kv_stride_tok, int32_t page_size,
                                 const int32_t* block_tables, int64_t bt_stride,
                                 int32_t pages_per_seq, const float* k_scale, const float* v_scale,
                                 const int32_t* seq_lens, int32_t batch, const float* sinks,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 float scale, int32_t split_size, int32_t num_splits,
                                 float* part_o, float* part_m, float* part_d, void* stream) {
  g_err[0] = '\0';
  if ((k_scale == nullptr) != (v_scale == nullptr))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given or both be null");
  if (page_size <= 0) return fail(SINK_ATTN_EINVAL, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
  if (pages_per_seq < 0) return fail(SINK_ATTN_EINVAL, "pages_per_seq must be >= 0");
  const int64_t max_ctx = static_cast<int64_t>(pages_per_seq) * page_size;
  if (max_ctx > 0x7fffffff) return fail(SINK_ATTN_EUNSUPPORTED, "pages_per_seq * page_size exceeds 2^31");
  return decode_multi_split(q, q_stride_b, q_stride_tok, q_stride_head, q_len, k_pages, v_pages,
                            page_stride, kv_stride_head, kv_stride_tok, k_scale, v_scale,
                            block_tables, bt_stride, page_size, seq_lens, batch,
                            static_cast<int32_t>(max_ctx), sinks, num_q_heads, num_kv_heads,
                            head_dim, scale, split_size, num_splits, part_o, part_m, part_d,
                            stream);
}

int sink_attn_decode_split(const void* q, int64_t q_stride_b, int64_t q_stride_head,
                           const void* k_cache, const void* v_cache, int64_t kv_stride_b,
                           int64_t kv_stride_head, int64_t kv_stride_tok,
                           const int32_t* seq_lens, int32_t batch, int32_t max_ctx,
                           const float* sinks, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, float scale, int32_t split_size,
                           int32_t num_splits, float* part_o, float* part_m,
                           float* part_d, void* stream) {
  // one new token per request: the multi-token form with q_len = 1
  return sink_attn_decode_multi_split(q, q_stride_b, 0, q_stride_head, 1, k_cache, v_cache,
                                      kv_stride_b, kv_stride_head, kv_stride_tok, seq_lens, batch,
                                      max_ctx, sinks, num_q_heads, num_kv_heads, head_dim, scale,
                                      split_size, num_splits, part_o, part_m, part_d, stream);
}

int32_t sink_attn_decode_split_size(int32_t batch, int32_t max_ctx, int32_t q_len,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    const int32_t* seq_lens_host) {
  g_err[0] = '\0';
  if (batch < 0 || max_ctx < 0) return fail(SINK_ATTN_EINVAL, "batch and max_ctx must be >= 0");
  if (q_len < 1) return fail(SINK_ATTN_EINVAL, "q_len must be >= 1 (got %d)", q_len);
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  // with the lengths: their longest, and whether they are (nearly) equal
  int max_len = max_ctx;
  bool uniform = false;
  if (seq_lens_host != nullptr && batch > 0) {
    int64_t total = 0;
    int longest = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t len = seq_lens_host[b];
      if (len < 0 || len > max_ctx)
        return fail(SINK_ATTN_EINVAL, "seq_lens_host[%d] = %d is outside [0, max_ctx = %d]", b, len,
                    max_ctx);
      total += len;
      longest = len > longest ? len : longest;
    }
    max_len = longest;
    uniform = longest > 0 && 10 * total >= 9 * static_cast<int64_t>(batch) * longest;
  }
  int device = 0, cus = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  const int64_t ncols = static_cast<int64_t>(q_len) * (num_q_heads / num_kv_heads);
  const int cols_per_block = 16 * sinkattn::decode_column_blocks(
      static_cast<int>(ncols > 0x7fffffff ? 0x7fffffff : ncols), head_dim);
  const int64_t slices = (ncols + cols_per_block - 1) / cols_per_block;
  return sinkattn::decode_split_size(static_cast<int64_t>(batch) * num_kv_heads * slices, max_len,
                                     uniform, head_dim, cus);
}

int sink_attn_merge_states(const float* part_o, const float* part_m, const float* part_d,
                           int32_t batch, int32_t num_q_heads, int32_t num_splits,
                           int32_t head_dim, void* o, int64_t o_stride_b,
                           int64_t o_stride_head, float* lse, void* stream) {
  g_err[0] = '\0';
  if (batch < 0) return fail(SINK_ATTN_EINVAL, "batch must be >= 0");
  if (num_q_heads <= 0) return fail(SINK_ATTN_EINVAL, "num_q_heads must be positive");
  if (num_splits <= 0) return fail(SINK_ATTN_EINVAL, "num_splits must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(SINK_ATTN_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  if (batch == 0) return SINK_ATTN_OK;
  if (!part_o || !part_m || !part_d || !o) return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  if (!aligned(o, 16)) return fail(SINK_ATTN_EINVAL, "o must be 16-byte aligned");
  if (!aligned(part_o, 4) || !aligned(part_m, 4) || !aligned(part_d, 4) || (lse && !aligned(lse, 4)))
    return fail(SINK_ATTN_EINVAL, "fp32 buffers must be 4-byte aligned");
  if (!stride_ok(o_stride_b) || !stride_ok(o_stride_head))
    return fail(SINK_ATTN_EINVAL, "strides must be non-negative multiples of 8 elements");
  const int64_t rows = static_cast<int64_t>(batch) * num_q_heads;
  if (rows > 0x7fffffff / 2) return fail(SINK_ATTN_EUNSUPPORTED, "problem too large for one launch");

  sinkattn::MergeArgs a{};
  a.part_o = part_o;
  a.part_m = part_m;
  a.part_d = part_d;
  a.o = static_cast<uint16_t*>(o);
  a.o_sb = o_stride_b;
  a.o_st = 0;
  a.o_sh = o_stride_head;
  a.lse = lse;
  a.rows = static_cast<int32_t>(rows);
  a.q_len = 1;
  a.num_q_heads = num_q_heads;
  a.num_splits = num_splits;
  return launched(sinkattn::launch_merge(a, head_dim, static_cast<hipStream_t>(stream)), "merge_states");
}

// KV append into bf16 caches (k_scale == nullptr: a copy) or FP8 E4M3 caches.
static int kv_append(const void* k_new, const void* v_new, int64_t new_stride_tok,
                     int64_t new_stride_head, const int32_t* cu_seqlens_new,
                     const int32_t* cache_pos, int32_t num_seqs, int32_t max_new, void* k_cache,
                     void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                     int64_t kv_stride_tok, const float* k_scale, const float* v_scale,
                     const int32_t* block_tables, int64_t bt_stride, int32_t page_size,
                     int32_t max_ctx, int32_t num_kv_heads, int32_t head_dim, void* stream) {
  const bool paged = page_size != 0;
  int page_shift = 0;
  if (paged) {
    if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
      return fail(SINK_ATTN_EINVAL, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
    while ((1 << page_shift) < page_size) ++page_shift;
    if (bt_stride < 0) return fail(SINK_ATTN_EINVAL, "block_tables row stride must be >= 0");
  }
  if (num_seqs < 0 || max_new < 0 || max_ctx < 0)
    return fail(SINK_ATTN_EINVAL, "num_seqs, max_new and max_ctx must be >= 0");
  if (num_kv_heads <= 0) return fail(SINK_ATTN_EINVAL, "num_kv_heads must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(SINK_ATTN_EUNSUPPORTED, "head_dim %d is not supported (64 or 128)", head_dim);
  if (num_seqs == 0 || max_new == 0 || max_ctx == 0) return SINK_ATTN_OK;
  if (!k_new || !v_new || !cu_seqlens_new || !cache_pos || !k_cache || !v_cache ||
      (paged && !block_tables))
    return fail(SINK_ATTN_EINVAL, "a required pointer is null");
  if (paged && !aligned(block_tables, 4))
    return fail(SINK_ATTN_EINVAL, "block_tables must be 4-byte aligned");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(SINK_ATTN_EINVAL, "k_new, v_new and the caches must be 16-byte aligned");
  if (!aligned(cu_seqlens_new, 4) || !aligned(cache_pos, 4))
    return fail(SINK_ATTN_EINVAL, "cu_seqlens_new and cache_pos must be 4-byte aligned");
  if (!stride_ok(new_stride_tok) || !stride_ok(new_stride_head) || !stride_ok(kv_stride_b) ||
      !stride_ok(kv_stride_head) || !stride_ok(kv_stride_tok))
    return fail(SINK_ATTN_EINVAL, "strides must be non-negative multiples of 8 elements");
  if (k_new == k_cache || v_new == v_cache || k_cache == v_cache)
    return fail(SINK_ATTN_EINVAL, "the caches must not alias each other or the new rows");
  if ((k_scale || v_scale) && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given, 4-byte aligned");

  const int tpb = sinkattn::kv_append_tokens_per_block(head_dim);
  const int64_t token_blocks = (static_cast<int64_t>(max_new) + tpb - 1) / tpb;
  const int64_t num_blocks = static_cast<int64_t>(num_seqs) * num_kv_heads * token_blocks;
  if (num_blocks > 0x7fffffff) return fail(SINK_ATTN_EUNSUPPORTED, "problem too large for one launch");

  sinkattn::KvAppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.new_st = new_stride_tok;
  a.new_sh = new_stride_head;
  a.cu_seqlens_new = cu_seqlens_new;
  a.cache_pos = cache_pos;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = paged ? block_tables : nullptr;
  a.bt_stride = bt_stride;
  a.page_shift = page_shift;
  a.kv_sb = kv_stride_b;
  a.kv_sh = kv_stride_head;
  a.kv_st = kv_stride_tok;
  a.max_ctx = max_ctx;
  a.num_kv_heads = num_kv_heads;
  a.token_blocks = static_cast<int32_t>(token_blocks);
  return launched(sinkattn::launch_kv_append(a, head_dim, num_blocks, static_cast<hipStream_t>(stream)),
                  "kv_append");
}


int sink_attn_kv_append(const void* k_new, const void* v_new, int64_t new_stride_tok,
                        int64_t new_stride_head, const int32_t* cu_seqlens_new,
                        const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                        void* k_cache, void* v_cache, int64_t kv_stride_b, int64_t kv_stride_head,
                        int64_t kv_stride_tok, int32_t max_ctx, int32_t num_kv_heads,
                        int32_t head_dim, void* stream) {
  g_err[0] = '\0';
  return kv_append(k_new, v_new, new_stride_tok, new_stride_head, cu_seqlens_new, cache_pos,
                   num_seqs, max_new, k_cache, v_cache, kv_stride_b, kv_stride_head,
                   kv_stride_tok, nullptr, nullptr, nullptr, 0, 0, max_ctx, num_kv_heads, head_dim,
                   stream);
}

int sink_attn_kv_append_fp8(const void* k_new, const void* v_new, int64_t new_stride_tok,
                            int64_t new_stride_head, const int32_t* cu_seqlens_new,
                            const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                            void* k_cache, void* v_cache, int64_t kv_stride_b,
                            int64_t kv_stride_head, int64_t kv_stride_tok, const float* k_scale,
                            const float* v_scale, int32_t max_ctx, int32_t num_kv_heads,
                            int32_t head_dim, void* stream) {
  g_err[0] = '\0';
  if (!k_scale || !v_scale) return fail(SINK_ATTN_EINVAL, "k_scale and v_scale are required");
  return kv_append(k_new, v_new, new_stride_tok, new_stride_head, cu_seqlens_new, cache_pos,
                   num_seqs, max_new, k_cache, v_cache, kv_stride_b, kv_stride_head,
                   kv_stride_tok, k_scale, v_scale, nullptr, 0, 0, max_ctx, num_kv_heads, head_dim,
                   stream);
}

int sink_attn_kv_append_paged(const void* k_new, const void* v_new, int64_t new_stride_tok,
                              int64_t new_stride_head, const int32_t* cu_seqlens_new,
                              const int32_t* cache_pos, int32_t num_seqs, int32_t max_new,
                              void* k_pages, void* v_pages, int64_t page_stride,
                              int64_t kv_stride_head, int64_t kv_stride_tok, int32_t page_size,
                              const int32_t* block_tables, int64_t bt_stride,
                              int32_t pages_per_seq, const float* k_scale, const float* v_scale,
                              int32_t num_kv_heads, int32_t head_dim, void* stream) {
  g_err[0] = '\0';
  if ((k_scale == nullptr) != (v_scale == nullptr))
    return fail(SINK_ATTN_EINVAL, "k_scale and v_scale must both be given or both be null");
  if (page_size <= 0) return fail(SINK_ATTN_EINVAL, "page_size must be a power of two in [16, 2^20] (got %d)", page_size);
  if (pages_per_seq < 0) return fail(SINK_ATTN_EINVAL, "pages_per_seq must be >= 0");
  const int64_t max_ctx = static_cast<int64_t>(pages_per_seq) * page_size;
  if (max_ctx > 0x7fffffff) return fail(SINK_ATTN_EUNSUPPORTED, "pages_per_seq * page_size exceeds 2^31");
  return kv_append(k_new, v_new, new_stride_tok, new_stride_head, cu_seqlens_new, cache_pos,
                   num_seqs, max_new, k_pages, v_pages, page_stride, kv_stride_head,
                   kv_stride_tok, k_scale, v_scale, block_tables, bt_stride, page_size,
                   static_cast<int32_t>(max_ctx), num_kv_heads, head_dim, stream);
}

}  // extern "C"
