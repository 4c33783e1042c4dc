// Split-KV decode with a per-head sink logit and the merge of chunk states, gfx950.
//
// Method: "GPT-OSS on day 0" (Perplexity blog), section "Kernels for GPT-OSS /
// Sink-Attention" -- attention is parallelised over heads and over the KV
// length; the running maximum is seeded with the sink and only the first
// chunk of a split key range may carry it.  "Hosting Qwen on Blackwell",
// section "Deployment on GB200 NVL72": the KV cache is HND (heads leading,
// the tokens of one head contiguous); section "Decoders": decode is bound by
// memory traffic, so the kernel is built to stream the cache once.
//
// decode_split_kernel: one workgroup (4 waves) per (request b, KV head g,
// 16-head slice of g's query heads, chunk c).  The K/V of the chunk are read
// exactly once and serve every query head of the group.  Each wave takes 64
// consecutive keys per step; the 4 waves cover 256 keys per step.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 d loaded
//     straight from HBM (16 bytes per lane, whole 128-byte rows per 8 lanes),
//     B = Q^T of up to 16 heads (padding columns are zero).
//   * the softmax state is per lane (column = head); row max / sum reduce over
//     the four 16-lane rows with permlane16/32 swaps.
//   * O^T += V^T P^T on the same MFMA; V goes through a per-wave LDS tile
//     written transposed, P^T comes straight from the S^T accumulators.
//   * at the end the 4 waves' states are merged through LDS and the chunk's
//     (o / d, m, d) is written in fp32.  Only wave 0 of chunk 0 seeds the sink.
// merge_kernel: one wave per (b, h) row, lane = d; log-sum-exp weighted sum of
// the chunk states, rounded to bf16.
#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaveKeys = 64;                 // keys per wave per step
constexpr int kStepKeys = 4 * kWaveKeys;      // keys per workgroup per step

// Position of key k (0..63) in a transposed-V row: within each 32-key half,
// the 8 keys one 16x16x32 MFMA lane row-group b consumes
// ({4b..4b+3, 16+4b..16+4b+3}) are made contiguous.
__device__ __forceinline__ int vt_pos16(int k) {
  return (k & 32) + (((k >> 2) & 3) << 3) + (((k >> 4) & 1) << 2) + (k & 3);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int DC = D / 8;                                // 16-byte chunks per row
  constexpr int VIT = (kWaveKeys / 2) * DC / 64;           // V items per lane
  constexpr int VT = D * kWaveKeys;                        // elements of one wave's V^T tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * VT];

  int unit = blockIdx.x;
  const int c = unit % a.num_splits;
  unit /= a.num_splits;
  const int hs = unit % a.head_slices;
  unit /= a.head_slices;
  const int g = unit % a.num_kv_heads;
  const int b = unit / a.num_kv_heads;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;           // query head of the slice this lane serves
  const int lgrp = lane >> 4;          // 16-lane row group 0..3
  const int h0 = g * a.group + hs * 16;
  const int nh = min(16, a.group - hs * 16);
  const bool hvalid = col < nh;
  const int h = h0 + (hvalid ? col : 0);

  const int len = a.seq_lens[b];
  const int lo = c * a.split_size;
  const int hi = min(lo + a.split_size, len);
  const int n = max(hi - lo, 0);
  const int nsteps = (n + kStepKeys - 1) / kStepKeys;

  // Q^T fragments: column = head, k = d
  u32x4_t qf[D / 32];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh + 8 * lgrp;
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc) {
      u32x4_t t = load16(qp + 32 * cc);
      qf[cc] = hvalid ? t : u32x4_t{0, 0, 0, 0};
    }
  }

  // state: the sink seeds wave 0 of chunk 0 only, counted once (row group 0)
  const float sink = hvalid ? a.sinks[h] : -INFINITY;
  const bool seeded = (c == 0) && (wave == 0);
  float m = seeded ? sink * kLog2e : -INFINITY;
  float l = (seeded && lgrp == 0 && sink != -INFINITY) ? 1.f : 0.f;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = f32x4_t{};

  const uint16_t* kbase = a.k_cache + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const uint16_t* vbase = a.v_cache + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  uint16_t* vt = smem + wave * VT;

  for (int step = 0; step < nsteps; ++step) {
    const int k0 = lo + step * kStepKeys + wave * kWaveKeys;   // first key of this wave

    // K fragments (A operand: row = key, k = d) straight from the cache
    u32x4_t kf[4][D / 32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = k0 + kb * 16 + col;
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc)
        kf[kb][cc] = key < hi ? load16(kbase + (int64_t)key * a.kv_st + 32 * cc + 8 * lgrp)
                              : u32x4_t{0, 0, 0, 0};
    }
    // V rows, two consecutive keys x 8 d per item
    u32x4_t vr[VIT][2];
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = lane + 64 * i;
      const int key = k0 + 2 * (it / DC);
      const int ch = it % DC;
      vr[i][0] = key < hi ? load16(vbase + (int64_t)key * a.kv_st + ch * 8) : u32x4_t{0, 0, 0, 0};
      vr[i][1] = key + 1 < hi ? load16(vbase + (int64_t)(key + 1) * a.kv_st + ch * 8)
                              : u32x4_t{0, 0, 0, 0};
    }

    // S^T = K Q^T
    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{};
#pragma unroll
      for (int cc = 0; cc < D / 32; ++cc) s[kb] = mfma_16x16x32(kf[kb][cc], qf[cc], s[kb]);
    }

    // V -> transposed LDS tile (this wave's region)
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = lane + 64 * i;
      const int key = 2 * (it / DC);
      const int ch = it % DC;
      const int pos = vt_pos16(key);
      const int pch = pos >> 3, within = pos & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = ch * 8 + e;
        const uint32_t x = vr[i][0][e >> 1], y = vr[i][1][e >> 1];
        const uint32_t w = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
        *reinterpret_cast<uint32_t*>(vt + d * kWaveKeys + ((pch ^ vt_swizzle(d)) * 8) + within) = w;
      }
    }

    // mask keys past the chunk end
    if (k0 + kWaveKeys > hi) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + kb * 16 + 4 * lgrp + i >= hi) s[kb][i] = -INFINITY;
    }

    // online softmax update (log2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair16_max(mx);
    mx = pair32_max(mx);
    const float m_new = fmaxf(m, mx * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(s[kb][i] * a.scale_log2 - m_use);
        s[kb][i] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;

    __syncthreads();   // transposed V visible to the whole wave

    // O^T += V^T P^T, 32 keys per MFMA
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4_t pf;
      pf[0] = pack_bf16x2(s[2 * j][0], s[2 * j][1]);
      pf[1] = pack_bf16x2(s[2 * j][2], s[2 * j][3]);
      pf[2] = pack_bf16x2(s[2 * j + 1][0], s[2 * j + 1][1]);
      pf[3] = pack_bf16x2(s[2 * j + 1][2], s[2 * j + 1][3]);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int d = db * 16 + col;
        const int ch = (4 * j + lgrp) ^ vt_swizzle(d);
        acc[db] = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(vt + d * kWaveKeys + ch * 8),
                                pf, acc[db]);
      }
    }
    __syncthreads();   // V^T reads done before the next step overwrites it
  }

  // ---- merge the four waves' states through LDS ------------------------------
  l = pair16_sum(l);
  l = pair32_sum(l);
  float* red = reinterpret_cast<float*>(smem);
  float* red_m = red;                 // [4][16]
  float* red_l = red + 64;            // [4][16]
  float* red_o = red + 128;           // [4][D][16]
  if (lgrp == 0) {
    red_m[wave * 16 + col] = m;
    red_l[wave * 16 + col] = l;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[(wave * D + db * 16 + 4 * lgrp + i) * 16 + col] = acc[db][i];
  __syncthreads();

  for (int item = tid; item < nh * D; item += kThreads) {
    const int qh = item / D, d = item % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * 16 + qh]);
    float wsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(red_m[w * 16 + qh] - M);
        wsum += red_l[w * 16 + qh] * f;
        o += red_o[(w * D + d) * 16 + qh] * f;
      }
    }
    const int64_t row = ((int64_t)b * a.num_q_heads + h0 + qh) * a.num_splits + c;
    a.part_o[row * D + d] = wsum > 0.f ? o / wsum : 0.f;
    if (d == 0) {
      a.part_m[row] = M == -INFINITY ? -INFINITY : M * kLn2;
      a.part_d[row] = wsum;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const int ns = a.num_splits;
  const float* pm = a.part_m + (int64_t)row * ns;
  const float* pd = a.part_d + (int64_t)row * ns;
  const float* po = a.part_o + (int64_t)row * ns * D;
  float M = -INFINITY;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, pm[c]);
  float W = 0.f;
  float acc[D / 64] = {};
  if (M != -INFINITY) {
    for (int c = 0; c < ns; ++c) {
      const float mc = pm[c];
      const float w = mc == -INFINITY ? 0.f : pd[c] * fast_exp2((mc - M) * kLog2e);
      W += w;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) acc[j] += w * po[(int64_t)c * D + lane + 64 * j];
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int b = row / a.num_q_heads, h = row % a.num_q_heads;
  uint16_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const __bf16 v = (__bf16)(acc[j] * inv);
    op[lane + 64 * j] = __builtin_bit_cast(uint16_t, v);
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = W > 0.f ? M + __logf(W) : -INFINITY;
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int64_t num_blocks,
                               hipStream_t stream) {
  const dim3 grid((unsigned)num_blocks), block(kThreads);
  if (head_dim == 64)
    hipLaunchKernelGGL(decode_split_kernel<64>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<128>, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + 3) / 4)), block(kThreads);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
