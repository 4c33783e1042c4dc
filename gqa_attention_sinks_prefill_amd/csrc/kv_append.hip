// Append new tokens' K and V to per-request HND caches, gfx950.
//
// "Hosting Qwen on Blackwell" (Perplexity blog), section "Deployment on GB200
// NVL72": KV caches are kept in HND order -- heads leading, the tokens of one
// head contiguous -- while the tokens that a prefill or decode step produces
// arrive token-major (one row of all KV heads per token, as the QKV
// projection writes them).  Sections "Prefillers" / "Decoders": prefill fills
// the caches that the decoders then stream.  This kernel moves a batch of new
// tokens into their requests' caches: new token t of request b, KV head g,
// goes to cache slot (b, g, cache_pos[b] + t).
//
// It is a pure copy (bytes in = bytes out, bit-exact) into bf16 caches, or a
// quantization into FP8 E4M3 caches with a scale per KV head (the code of x is
// fp32(x) * (1 / scale) rounded to nearest even, saturated at +-448).  Bound by HBM: one
// workgroup per (request, KV head, block of new tokens); each thread moves one
// 16-byte chunk of K and of V, the chunk index fastest so that the stores of
// consecutive tokens of one head form one contiguous run.  Tokens
// past the request's count or past the cache end are skipped (device-side
// lengths cannot be checked on the host).
#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kThreads = 256;
// Token rows per thread.  One row per thread with non-temporal loads and
// stores (nothing re-reads the new rows or the slots just written) measured
// 5.6 TB/s moved for 64 x 1024 new rows of 8 heads (d 64), against 4.7 TB/s
// for four rows per thread with plain accesses (FP8 caches: 5.0 vs 4.4).
constexpr int kPasses = 1;
constexpr float kE4M3Max = 448.f;             // largest finite E4M3 value

// Eight values -> eight E4M3 codes of a cache with dequantization scale
// 1 / inv: fp32(x) * inv, saturated to +-448, rounded to nearest even.
__device__ __forceinline__ u32x2_t quantize8(const u32x4_t& bf, float inv) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(bf[i] << 16) * inv;
    f[2 * i + 1] = __uint_as_float(bf[i] & 0xffff0000u) * inv;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)     // a NaN stays NaN (a NaN code)
    f[i] = __builtin_isnan(f[i]) ? f[i] : fminf(fmaxf(f[i], -kE4M3Max), kE4M3Max);
  u32x2_t r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w], f[4 * w + 1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2], f[4 * w + 3], v, true);
    r[w] = (uint32_t)v;
  }
  return r;
}

template <int D, bool F8, bool PG>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(KvAppendArgs a) {
  constexpr int DC = D / 8;                   // 16-byte chunks per bf16 token row
  constexpr int TPP = kThreads / DC;          // tokens per pass
  constexpr int TB = TPP * kPasses;           // tokens per workgroup
  int unit = blockIdx.x;
  const int tb = unit % a.token_blocks;
  unit /= a.token_blocks;
  const int g = unit % a.num_kv_heads;
  const int b = unit / a.num_kv_heads;

  const int start = a.cu_seqlens_new[b];
  const int n = a.cu_seqlens_new[b + 1] - start;
  const int64_t pos = a.cache_pos[b];
  const int c = threadIdx.x % DC;
  const int t0 = tb * TB + threadIdx.x / DC;
  const int64_t cache_row = (PG ? 0 : (int64_t)b * a.kv_sb) + (int64_t)g * a.kv_sh;

  u32x4_t kr[kPasses], vr[kPasses];
  bool ok[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int t = t0 + p * TPP;
    ok[p] = t < n && pos >= 0 && pos + t < a.max_ctx;
    if (ok[p]) {
      const int64_t src = (int64_t)(start + t) * a.new_st + (int64_t)g * a.new_sh + 8 * c;
      kr[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new + src));
      vr[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new + src));
    }
  }
  float k_inv = 0.f, v_inv = 0.f;
  if constexpr (F8) {
    k_inv = 1.0f / a.k_scale[g];              // correctly rounded division
    v_inv = 1.0f / a.v_scale[g];
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (ok[p]) {
      const int64_t slot = pos + t0 + p * TPP;
      int64_t dst;
      if constexpr (PG) {   // page block_tables[b][slot / P], row slot % P
        const int32_t page = a.block_tables[(int64_t)b * a.bt_stride + (slot >> a.page_shift)];
        dst = (int64_t)page * a.kv_sb + cache_row + (slot & ((1 << a.page_shift) - 1)) * a.kv_st + 8 * c;
      } else {
        dst = cache_row + slot * a.kv_st + 8 * c;
      }
      if constexpr (F8) {
        __builtin_nontemporal_store(quantize8(kr[p], k_inv), reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(a.k_cache) + dst));
        __builtin_nontemporal_store(quantize8(vr[p], v_inv), reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(a.v_cache) + dst));
      } else {
        __builtin_nontemporal_store(kr[p], reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.k_cache) + dst));
        __builtin_nontemporal_store(vr[p], reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.v_cache) + dst));
      }
    }
  }
}

}  // namespace

int kv_append_tokens_per_block(int head_dim) { return kThreads / (head_dim / 8) * kPasses; }

hipError_t launch_kv_append(const KvAppendArgs& a, int head_dim, int64_t num_blocks,
                            hipStream_t stream) {
  const dim3 grid((unsigned)num_blocks), block(kThreads);
  const int kind = (a.k_scale != nullptr ? 1 : 0) + (a.block_tables != nullptr ? 2 : 0);
  switch (kind + (head_dim == 64 ? 0 : 4)) {
    case 0: hipLaunchKernelGGL((kv_append_kernel<64, false, false>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((kv_append_kernel<64, true, false>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((kv_append_kernel<64, false, true>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((kv_append_kernel<64, true, true>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((kv_append_kernel<128, false, false>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((kv_append_kernel<128, true, false>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((kv_append_kernel<128, false, true>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((kv_append_kernel<128, true, true>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace sinkattn
