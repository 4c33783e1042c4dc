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
//   * K and V tiles (64 keys) are copied HBM -> LDS by buffer->LDS DMA, row
//     major with XOR-swizzled 16-byte chunks (k_swz / v_swz below); the copies
//     of the next tiles run during the current tile's math and need no
//     registers.  Reads past the sequence end return zeros.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T in
//     registers): each lane owns one query row, so the row max needs a single
//     cross-lane step (lanes l and l^32).
//   * O^T += V^T P^T: P^T is the S^T accumulator, reused as the B operand with
//     the contraction index permuted; V^T operands come from the row-major V
//     tile through the transposing LDS read, in the same permutation.
//   * The softmax denominator is accumulated on the matrix pipe as well
//     (a ones row times P^T), so per score the vector ALU does only the max,
//     one fma + exp2 and half a bf16 pack.
//   * Software pipeline: iteration j issues the QK^T MFMAs of tile j+1 next to
//     the exponentials and P.V MFMAs of tile j.
//   * Lazy rescaling: the running maximum m only moves when a row's tile max
//     exceeds it by more than kRescaleLog2 (log2 units); until then the
//     weights exp2(x - m) stay below 2^kRescaleLog2, and O and the denominator
//     share the same stale m, so o = O / d is unchanged.  One wave-uniform
//     branch per tile.
//   * Only the last tiles of a row block need the causal / length mask, applied
//     under a wave-uniform branch together with the tile's row max.
//   * Block order: heaviest causal row tiles first, and the head groups that
//     share a KV head are kept on one XCD (workgroups go round-robin over the
//     8 XCDs), so each XCD's L2 holds the K/V of its own heads.
#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBlockN = 64;        // keys per tile
constexpr int kThreads = 256;
constexpr float kRescaleLog2 = 8.f;
constexpr uint32_t kOnesBf16x2 = 0x3f803f80u;   // two bf16 1.0

// Chunk swizzles of the row-major K and V tiles.  K is read 16 bytes per lane
// down 32 consecutive rows: XOR with row % 8 spreads any 8 rows over all
// eight 16-byte bank groups.  V is read 8 bytes per lane by the transposing
// read, four consecutive rows x two adjacent chunks per 16-lane group: XOR with
// 2 * (row % 4) gives those eight chunk reads eight distinct bank groups.
__device__ __forceinline__ int k_swz(int row) { return row & 7; }
__device__ __forceinline__ int v_swz(int row) { return 2 * (row & 3); }

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void prefill_kernel(PrefillArgs a) {
  constexpr int RB = 4 / HPW;            // 32-row blocks per workgroup
  constexpr int ROWS = 32 * RB;
  constexpr int DC = D / 8;              // 16-byte chunks per key row
  constexpr int KT = kBlockN * D;        // elements of one K or V tile
  constexpr int DMA = kBlockN * DC / kThreads;   // 16-byte DMA slots per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * KT];   // K0 K1 V0 V1

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
  const int ntiles = (kv_end + kBlockN - 1) / kBlockN;
  // leading tiles that no row of this workgroup needs masked
  const int nfull = min(a.causal ? (q0 + 1) / kBlockN : ntiles, len / kBlockN);

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

  // ---- K / V buffer resources over the visible keys -------------------------
  const int k_st2 = (int)(a.k_st * 2), v_st2 = (int)(a.v_st * 2);   // bytes per token
  const auto krs = make_rsrc(a.k + (int64_t)start * a.k_st + (int64_t)g * a.k_sh,
                             kv_end > 0 ? (kv_end - 1) * k_st2 + 2 * D : 0);
  const auto vrs = make_rsrc(a.v + (int64_t)start * a.v_st + (int64_t)g * a.v_sh,
                             kv_end > 0 ? (kv_end - 1) * v_st2 + 2 * D : 0);

  // DMA: thread t's i-th copy fills LDS slot (16 bytes) s = 64*(4i + wave) + lane
  // of a tile, i.e. key row s / DC, physical chunk s % DC.  K rows hold the
  // logical chunk (s % DC) ^ k_swz(row), V rows (s % DC) ^ v_swz(row).
  int k_goff[DMA], v_goff[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int s = 64 * (4 * i + wave) + lane, key = s / DC;
    k_goff[i] = key * k_st2 + ((s % DC) ^ k_swz(key)) * 16;
    v_goff[i] = key * v_st2 + ((s % DC) ^ v_swz(key)) * 16;
  }
  auto dma_k = [&](int kt, int buf) {
    uint16_t* dst = smem + buf * KT + wave * 512;
    const int off = kt * kBlockN * k_st2;
#pragma unroll
    for (int i = 0; i < DMA; ++i) buffer_load16_lds(krs, dst + i * 2048, k_goff[i] + off);
  };
  auto dma_v = [&](int kt, int buf) {
    uint16_t* dst = smem + (2 + buf) * KT + wave * 512;
    const int off = kt * kBlockN * v_st2;
#pragma unroll
    for (int i = 0; i < DMA; ++i) buffer_load16_lds(vrs, dst + i * 2048, v_goff[i] + off);
  };

  // LDS read offsets (elements).  K (ds_read_b128): row kb*32 + lrow, logical
  // chunk 2c + lhalf.  V^T (transposing read): lane i of a 16-lane group
  // addresses key row 16u + 8t + 4*lhalf + (i >> 2), d = 32db + 16*((lane>>4)&1)
  // + 4*(i & 3).
  int k_roff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_roff[c] = lrow * D + (((2 * c + lhalf) ^ k_swz(lrow)) * 8);
  int v_roff[2];
  {
    const int i = lane & 15, gi = (lane >> 4) & 1;
    const int row = 4 * lhalf + (i >> 2);                 // key row within an 8-row group
#pragma unroll
    for (int dbp = 0; dbp < 2; ++dbp) {
      const int cl = 4 * dbp + 2 * gi + ((i & 3) >> 1);   // logical chunk for db = dbp
      v_roff[dbp] = row * D + ((cl ^ v_swz(row)) * 8) + 4 * (i & 1);
    }
  }
  auto qk = [&](int buf, f32x16_t (&s)[2]) {   // S^T = K Q^T for one tile
    const uint16_t* ks = smem + buf * KT;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        s[kb] = mfma_32x32x16(*reinterpret_cast<const u32x4_t*>(ks + k_roff[c & 3] + kb * 32 * D + (c >> 2) * 64),
                              qf[c], s[kb]);
    }
  };

  // ---- running state, seeded with the sink ---------------------------------
  // m: running maximum in log2 units (never below -FLT_MAX so that m - m stays
  // finite).  lsum: the denominator on the matrix pipe -- every element of
  // this 32x32 accumulator holds the sum for the lane's query column; it
  // starts at the sink's exp2(0) = 1.
  const float sink = a.sinks[h];
  const float c2 = a.scale_log2;
  float m = fmaxf(sink * kLog2e, -__FLT_MAX__);
  f32x16_t lsum;
  {
    const float l0 = sink != -INFINITY ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) lsum[i] = l0;
  }
  f32x16_t acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16_t{};
  const int lim = a.causal ? min(qrow, len - 1) : len - 1;   // last visible key
  const u32x4_t ones = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};

  f32x16_t sa[2], sb[2];

  // Mask (for tiles past nfull) and row max of a tile's scores, in log2 units.
  auto tile_max = [&](int jt, f32x16_t (&s)[2]) -> float {
    if (jt >= nfull) {
      const int key0 = jt * kBlockN + 4 * lhalf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + kb * 32 + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }
    float mx = max3f(s[0][0], s[0][1], s[0][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = max3f(mx, s[0][i], s[0][i + 1]);
    mx = max3f(mx, s[0][15], s[1][0]);
#pragma unroll
    for (int i = 1; i < 15; i += 2) mx = max3f(mx, s[1][i], s[1][i + 1]);
    mx = fmaxf(mx, s[1][15]);
    return pair32_max(mx) * c2;
  };

  // One tile: rescale check and exponentials + P.V of tile j from s_cur (whose
  // mask and max t were prepared by the previous step), QK^T of tile j+1 into
  // s_nxt, and at the end the mask and max of tile j+1 -- so that vector work
  // overlaps the last P.V MFMAs instead of stalling the matrix pipe.
  float t;
  auto step = [&](int j, f32x16_t (&s_cur)[2], f32x16_t (&s_nxt)[2]) {
    // copies of K(j+2) and V(j+1) run during this tile's math
    if (j + 2 < ntiles) dma_k(j + 2, j & 1);
    if (j + 1 < ntiles) dma_v(j + 1, (j + 1) & 1);
    // move m only past the rescale threshold
    if (__builtin_amdgcn_ballot_w64(t > m + kRescaleLog2) != 0) {
      const float m_new = fmaxf(m, t);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
#pragma unroll
      for (int i = 0; i < 16; ++i) lsum[i] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    // S of tile j+1 on MFMA, next to the exponentials and P.V of tile j
    qk((j + 1) & 1, s_nxt);
    const uint16_t* vt = smem + (2 + (j & 1)) * KT;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = u >> 1, base = 8 * (u & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(s_cur[kb][base + e], c2, -m));
      u32x4_t pf;
      pf[0] = pack_bf16x2(p[0], p[1]);
      pf[1] = pack_bf16x2(p[2], p[3]);
      pf[2] = pack_bf16x2(p[4], p[5]);
      pf[3] = pack_bf16x2(p[6], p[7]);
      lsum = mfma_32x32x16(ones, pf, lsum);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vp = vt + v_roff[db & 1] + 16 * u * D + (db >> 1) * 64;
        const u32x2_t lo = lds_read_tr16(vp);
        const u32x2_t hi = lds_read_tr16(vp + 8 * D);
        const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
        acc[db] = mfma_32x32x16(vf, pf, acc[db]);
      }
    }
    if (j + 1 < ntiles) t = tile_max(j + 1, s_nxt);
    wait_vmem();
    __syncthreads();
  };

  // ---- prologue: K(0), V(0), K(1) staged; S and max of tile 0 ----------------
  dma_k(0, 0);
  dma_v(0, 0);
  if (ntiles > 1) dma_k(1, 1);
  wait_vmem();
  __syncthreads();
  qk(0, sa);
  t = tile_max(0, sa);
  __syncthreads();          // K buffer 0 is refilled in iteration 0

  // ---- tiles, two per trip so the S buffers swap roles ------------------------
  int j = 0;
  for (; j + 2 <= ntiles; j += 2) {
    step(j, sa, sb);
    step(j + 1, sb, sa);
  }
  if (j < ntiles) step(j, sa, sb);

  // ---- epilogue: normalise, round to bf16, store ----------------------------
  const float lt = lsum[0];
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
