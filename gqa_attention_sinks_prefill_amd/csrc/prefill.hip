// Causal / non-causal varlen prefill with a per-head sink logit, gfx950.
//
// Method: "GPT-OSS on day 0" (Perplexity blog), section "Kernels for GPT-OSS /
// Sink-Attention" -- an online softmax whose running maximum starts at the
// head's sink and whose running denominator starts at exp(sink - max) = 1, so
// the sink joins the softmax denominator without contributing a value row.
// Prefill is the compute-bound phase ("Hosting Qwen on Blackwell", section
// "Prefillers"), so both contractions run on bf16 MFMA with fp32 accumulation.
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   * a workgroup owns `HPW` query heads of one GQA group and 32*4/HPW query
//     rows of one sequence; wave w takes head (w % HPW) and row block w / HPW,
//     32 query rows each.  All waves share every K/V tile staged in LDS.
//   * S^T = K Q^T per 64-key tile on v_mfma_f32_32x32x16_bf16 (A = K from
//     LDS, B = Q^T held in registers), so each lane owns one query row and the
//     row max / row sum need only one cross-lane step (lanes l and l^32).
//   * O^T += V^T P^T, with P^T taken straight from the S^T accumulator
//     layout as the B operand (the contraction index is permuted consistently
//     in the transposed V tile), and V^T written into LDS once per tile.
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are
//     issued before the current tile's math.
//   * Block order: heaviest causal row tiles first, and the head groups that
//     share a KV head are kept on one XCD (workgroups go round-robin over the
//     8 XCDs), so each XCD's L2 holds the K/V of its own heads.
#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBlockN = 64;      // keys per tile
constexpr int kThreads = 256;

// Position of key `k` (0..63) inside a transposed-V row: within each 16-key
// block, the 8 keys a 32x32 MFMA lane half consumes ({0-3, 8-11} for lanes
// 0-31, {4-7, 12-15} for lanes 32-63) are made contiguous.
__device__ __forceinline__ int vt_pos32(int k) {
  int kk = k & 15;
  return (k & ~15) + (((kk >> 2) & 1) << 3) + ((kk >> 3) << 2) + (kk & 3);
}

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int RB = 4 / HPW;            // 32-row blocks per workgroup
  constexpr int ROWS = 32 * RB;
  constexpr int DC = D / 8;              // 16-byte chunks per K row
  constexpr int TILE = kBlockN * D;      // elements of one K (or V^T) tile
  constexpr int KCH = kBlockN * DC / kThreads;         // K chunks per thread
  constexpr int VIT = (kBlockN / 2) * DC / kThreads;   // (2 keys x 8 d) V items per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];

  // ---- work item -----------------------------------------------------------
  const int L = blockIdx.x;
  int hg, slot;
  if ((a.head_groups & 7) == 0) {
    const int per = a.head_groups >> 3;  // head groups per XCD
    hg = (L & 7) * per;
    slot = L >> 3;
    hg += slot % per;
    slot /= per;
  } else {
    hg = L % a.head_groups;
    slot = L / a.head_groups;
  }
  const int seq = slot % a.num_seqs;
  const int qtile = a.n_qtiles - 1 - slot / a.num_seqs;
  const int start = a.cu_seqlens[seq];
  const int len = a.cu_seqlens[seq + 1] - start;
  const int q0 = qtile * ROWS;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int h = hg * HPW + (wave % HPW);
  const int g = (hg * HPW) / a.group;
  const int w_row0 = q0 + (wave / HPW) * 32;
  const int qrow = w_row0 + lrow;        // position inside the sequence
  const bool qvalid = qrow < len;

  const int kv_end = a.causal ? min(q0 + ROWS, len) : len;
  const int w_kv_end = a.causal ? min(w_row0 + 32, len) : len;
  const int ntiles = (kv_end + kBlockN - 1) / kBlockN;

  // ---- Q^T fragments (B operand: column = query row, k = d) ---------------
  u32x4_t qf[D / 16];
  {
    const uint16_t* qp = a.q + (int64_t)(start + (qvalid ? qrow : 0)) * a.q_st +
                         (int64_t)h * a.q_sh + 8 * lhalf;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4_t t = load16(qp + 16 * c);
      qf[c] = qvalid ? t : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- running state, seeded with the sink ---------------------------------
  // m: running maximum in log2 units; l: this lane's share of the running
  // denominator (the sink's exp(0) = 1 is counted once, in lanes 0-31).
  const float sink = a.sinks[h];
  float m = sink * kLog2e;
  float l = (lhalf == 0 && sink != -INFINITY) ? 1.f : 0.f;
  f32x16_t acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16_t{};

  const uint16_t* kbase = a.k + (int64_t)start * a.k_st + (int64_t)g * a.k_sh;
  const uint16_t* vbase = a.v + (int64_t)start * a.v_st + (int64_t)g * a.v_sh;

  u32x4_t kreg[KCH];
  u32x4_t vreg[VIT][2];

  auto load_tile = [&](int kt) {
    const int key0 = kt * kBlockN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + kThreads * i;
      const int key = key0 + ci / DC;
      const int ch = ci % DC;
      kreg[i] = key < kv_end ? load16(kbase + (int64_t)key * a.k_st + ch * 8)
                             : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + kThreads * i;
      const int key = key0 + 2 * (it / DC);
      const int ch = it % DC;
      vreg[i][0] = key < kv_end ? load16(vbase + (int64_t)key * a.v_st + ch * 8)
                                : u32x4_t{0, 0, 0, 0};
      vreg[i][1] = key + 1 < kv_end ? load16(vbase + (int64_t)(key + 1) * a.v_st + ch * 8)
                                    : u32x4_t{0, 0, 0, 0};
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * 2 * TILE;
    uint16_t* vt = ks + TILE;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + kThreads * i;
      const int key = ci / DC;
      const int ch = ci % DC;
      *reinterpret_cast<u32x4_t*>(ks + key * D + ((ch ^ (key & 7)) * 8)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + kThreads * i;
      const int key = 2 * (it / DC);
      const int ch = it % DC;
      const int pos = vt_pos32(key);
      const int pch = pos >> 3, within = pos & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = ch * 8 + e;
        const uint32_t lo = vreg[i][0][e >> 1], hi = vreg[i][1][e >> 1];
        const uint32_t w = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                   : ((lo & 0xffffu) | (hi << 16));
        *reinterpret_cast<uint32_t*>(vt + d * kBlockN + ((pch ^ vt_swizzle(d)) * 8) + within) = w;
      }
    }
  };

  auto compute_tile = [&](int kt, int buf) {
    const int key0 = kt * kBlockN;
    if (key0 >= w_kv_end) return;          // tile lies past this wave's rows
    const uint16_t* ks = smem + buf * 2 * TILE;
    const uint16_t* vt = ks + TILE;

    // S^T = K Q^T for keys key0 .. key0+63 (two 32-key blocks)
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const int key = kb * 32 + lrow;
      const uint16_t* krow = ks + key * D;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const int ch = (2 * c + lhalf) ^ (key & 7);
        s[kb] = mfma_32x32x16(*reinterpret_cast<const u32x4_t*>(krow + ch * 8), qf[c], s[kb]);
      }
    }

    // mask: keys beyond the visible range of this lane's query row
    const bool need_mask = a.causal ? (key0 + kBlockN - 1 > w_row0) : (key0 + kBlockN > len);
    if (need_mask) {
      const int lim = a.causal ? min(qrow, len - 1) : len - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * lhalf + (i & 3);
          if (key > lim) s[kb][i] = -INFINITY;
        }
    }

    // online softmax update (log2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair32_max(mx);
    const float m_new = fmaxf(m, mx * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(s[kb][i] * a.scale_log2 - m_use);
        s[kb][i] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = u >> 1, base = 8 * (u & 1);
      u32x4_t pf;
      pf[0] = pack_bf16x2(s[kb][base + 0], s[kb][base + 1]);
      pf[1] = pack_bf16x2(s[kb][base + 2], s[kb][base + 3]);
      pf[2] = pack_bf16x2(s[kb][base + 4], s[kb][base + 5]);
      pf[3] = pack_bf16x2(s[kb][base + 6], s[kb][base + 7]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = db * 32 + lrow;
        const int ch = (2 * u + lhalf) ^ vt_swizzle(d);
        acc[db] = mfma_32x32x16(*reinterpret_cast<const u32x4_t*>(vt + d * kBlockN + ch * 8),
                                pf, acc[db]);
      }
    }
  };

  // ---- main loop: double-buffered K / V^T tiles -----------------------------
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);
    compute_tile(kt, buf);
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round to bf16, store ----------------------------
  const float lt = pair32_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qvalid) {
    uint16_t* op = a.o + (int64_t)(start + qrow) * a.o_st + (int64_t)h * a.o_sh + 4 * lhalf;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2_t w;
        w[0] = pack_bf16x2(acc[db][4 * i4 + 0] * inv, acc[db][4 * i4 + 1] * inv);
        w[1] = pack_bf16x2(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + db * 32 + 8 * i4) = w;
      }
    if (a.lse != nullptr && lhalf == 0)
      a.lse[(int64_t)(start + qrow) * a.num_q_heads + h] =
          lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int hpw, int64_t nb, hipStream_t st) {
  const dim3 grid((unsigned)nb), block(kThreads);
  switch (hpw) {
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

int prefill_heads_per_workgroup(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

int prefill_rows_per_workgroup(int group) { return 32 * 4 / prefill_heads_per_workgroup(group); }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int64_t num_blocks,
                          hipStream_t stream) {
  const int hpw = prefill_heads_per_workgroup(a.group);
  return head_dim == 64 ? launch_d<64>(a, hpw, num_blocks, stream)
                        : launch_d<128>(a, hpw, num_blocks, stream);
}

}  // namespace sinkattn
