// Kernel argument blocks and launchers behind the C ABI (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

struct PrefillArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint16_t* k;
  int64_t k_st, k_sh;
  const uint16_t* v;
  int64_t v_st, v_sh;
  const float* sinks;
  const int32_t* cu_seqlens;     // query tokens per sequence
  const int32_t* cu_seqlens_k;   // key tokens per sequence (== cu_seqlens for plain prefill)
  uint16_t* o;
  int64_t o_st, o_sh;
  float* lse;             // [T, Hq] or null
  int32_t num_seqs;
  int32_t n_qtiles;       // ceil(max_seqlen / rows per workgroup)
  int32_t num_q_heads;
  int32_t group;          // query heads per KV head
  int32_t head_groups;    // num_q_heads / heads per workgroup
  int32_t causal;
  float scale_log2;       // softmax scale * log2(e)
};

struct MergeArgs {
  const float* part_o;
  const float* part_m;
  const float* part_d;
  uint16_t* o;
  int64_t o_sb, o_st, o_sh;  // output strides: request, new token, head
  float* lse;
  int32_t rows;           // batch * q_len * num_q_heads
  int32_t q_len;          // new tokens per request (1 for plain decode)
  int32_t num_q_heads;
  int32_t num_splits;
  // Null: merge num_splits chunks per row.  Else the request lengths: merge
  // only the chunks that hold keys (chunk 0 at least) of each row's request.
  const int32_t* seq_lens;
  int32_t split_size;
};

struct DecodeArgs {
  const uint16_t* q;
  int64_t q_sb, q_st, q_sh;  // request, new-token and head strides
  const void* k_cache;       // bf16, or FP8 E4M3 codes when k_scale is set
  const void* v_cache;
  int64_t kv_sb, kv_sh, kv_st;  // in elements
  const float* k_scale;      // FP8 caches: dequantization scale per KV head (else null)
  const float* v_scale;
  const int32_t* block_tables;  // paged caches: [batch, >= pages per request] (else null)
  int64_t bt_stride;         // elements between block-table rows
  int64_t kv_sp;             // paged caches: elements between pages (kv_sb unused)
  int32_t page_shift;        // log2(page_size)
  const int32_t* seq_lens;
  const float* sinks;
  float* part_o;
  float* part_m;
  float* part_d;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // query heads per KV head
  int32_t q_len;          // new tokens per request (1 for plain decode)
  int32_t ncols;          // q_len * group columns: (new token, query head)
  int32_t head_slices;    // ceil(ncols / (16 * column blocks)): units per (b, g, chunk)
  int32_t batch;
  int32_t split_size;
  int32_t num_splits;
  float scale_log2;
  // Fused merge (else null): one arrival counter per (b, KV head, column
  // slice), zero before the launch and left zero after it; the workgroup that
  // completes a slice's last chunk merges its rows into merge.o / merge.lse.
  int32_t* counters;
  MergeArgs merge;
  // Chunks past a request's end write no state (a merge given the lengths
  // follows).
  int32_t skip_empty;
};


struct KvAppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_st, new_sh;  // token and head strides of the new rows
  const int32_t* cu_seqlens_new;
  const int32_t* cache_pos;
  void* k_cache;            // bf16, or FP8 E4M3 codes when k_scale is set
  void* v_cache;
  int64_t kv_sb, kv_sh, kv_st;  // in elements
  const float* k_scale;     // FP8 caches: dequantization scale per KV head (else null)
  const float* v_scale;
  const int32_t* block_tables;  // paged caches (else null); kv_sb is then the page stride
  int64_t bt_stride;
  int32_t page_shift;      // log2(page_size)
  int32_t max_ctx;         // slots per request (pages: table width * page_size)
  int32_t num_kv_heads;
  int32_t token_blocks;    // ceil(max_new / tokens per workgroup)
};

// Workgroup shape of the prefill kernel for a given GQA group size.
int prefill_heads_per_workgroup(int group);
int prefill_rows_per_workgroup(int group, int head_dim);

// one instantiation each (prefill_d64.hip, prefill_d128.hip)
hipError_t launch_prefill_d64(const PrefillArgs& a, int heads_per_wg, int64_t num_blocks,
                              hipStream_t stream);
hipError_t launch_prefill_d128(const PrefillArgs& a, int heads_per_wg, int64_t num_blocks,
                               hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int64_t num_blocks,
                          hipStream_t stream);
// Blocks of 16 columns one decode workgroup serves (1, 2, or up to 4 for head_dim 64).
int decode_column_blocks(int ncols, int head_dim);
// Waves (1, 2 or 4) that share one decode work unit.
int decode_waves_per_unit(int64_t num_units, int head_dim, int column_blocks);
// Tokens per chunk for split decode of `column_units` (request, KV head,
// column slice) triples over contexts of at most max_len tokens on `cus`
// compute units; `uniform`: the contexts are (nearly) all max_len long.
int decode_split_size(int64_t column_units, int max_len, bool uniform, int head_dim, int cus);
hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int64_t num_blocks,
                               hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream);
// fp32 elements of the device scratch array behind the no-allocation decode,
// and its address on the current device (looked up once per device).
constexpr int64_t kDecodeScratchFloats = int64_t(1) << 25;
hipError_t decode_scratch(float** out);
int kv_append_tokens_per_block(int head_dim);
hipError_t launch_kv_append(const KvAppendArgs& a, int head_dim, int64_t num_blocks,
                            hipStream_t stream);

}  // namespace sinkattn
