// Causal / non-causal varlen prefill with a per-head sink logit, gfx950, also
// in chunked form: a chunk of new queries per sequence against keys that hold
// the sequence's earlier tokens followed by the chunk ("Hosting Qwen on
// Blackwell", section "Prefillers", processes long inputs on prefill nodes;
// query i of a chunk of len_q at the end of len_k keys sees keys up to
// len_k - len_q + i).
//
// Method: "GPT-OSS on day 0" (Perplexity blog), section "Kernels for GPT-OSS /
// Sink-Attention" -- an online softmax whose running maximum starts at the
// head's sink and whose running denominator starts at exp(sink - max) = 1, so
// the sink joins the softmax denominator without contributing a value row.
// Prefill is the compute-bound phase ("Hosting Qwen on Blackwell", section
// "Prefillers"), so both contractions run on bf16 MFMA with fp32 accumulation.
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   * a workgroup owns `HPW` query heads of one GQA group and 4/HPW row groups
//     of one sequence; wave w takes head (w % HPW) and row group w / HPW of
//     32*QB query rows (QB 32-row blocks).  All waves share every K/V tile.
//     head_dim 64 uses QB = 2 with 32-key tiles, so each K operand and each
//     transposed V read feeds two MFMAs (half the LDS reads per MFMA);
//     head_dim 128 uses QB = 1 with 64-key tiles (registers).
//   * K and V tiles are copied HBM -> LDS by buffer->LDS DMA, row major with
//     XOR-swizzled 16-byte chunks (k_swz / v_swz below), into separate
//     double buffers; the copies of the next tiles run during the current
//     tile's math and need no registers.  Reads past the sequence end return
//     zeros.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T in
//     registers): each lane owns one query row per block.
//   * O^T += V^T P^T: P^T is the S^T accumulator layout reused as the B
//     operand with the contraction index permuted; V^T operands come from the
//     row-major V tile through the transposing LDS read in the same
//     permutation.
//   * No per-tile row max.  The exponentials use a stabiliser m that starts
//     at the sink's logit and moves (to the running row max, rescaling O and
//     the denominator) only when a tile's weights sum past kMaxTileSum --
//     detected after the exponentials, so the vector ALU does per score one
//     fma + exp2 and half a bf16 pack; the denominator is summed on the
//     matrix pipe (a 0/1 matrix times P^T on 16x16x32).  o = O / d does not
//     depend on m.
//   * Software pipeline: iteration j runs the QK^T MFMAs of tile j+1 next to
//     the exponentials of tile j; with head_dim 64 also the P.V MFMAs of tile
//     j-1 from operands held in registers, so that the matrix and vector
//     streams of one wave are independent until the stabiliser check.
//   * Only the last tiles of a row group need the causal / length mask, under
//     a wave-uniform branch.
//   * Block order: sequence by sequence, heaviest causal row tiles first
//     within a sequence, and the head groups that share a KV head are kept on
//     one XCD (workgroups go round-robin over the 8 XCDs): the workgroups
//     running together on an XCD then stream the K/V of one sequence and one
//     KV head, which its L2 holds.  (Round-robin over the sequences instead
//     had 16 packed sequences' K/V share each 4 MB L2: 8x the algorithmic
//     bytes fetched past L2, 13% slower at head_dim 128.)
#pragma once
// (The kernel template lives in this header; prefill_d64.hip and
// prefill_d128.hip instantiate one head_dim each, so that each can be built
// with its own code generation flags.)
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kThreads = 256;
constexpr float kMaxTileSum = 65536.f;   // 2^16: bound on a tile's weight sum per row

// Chunk swizzles of the row-major K and V tiles (DC 16-byte chunks per row).
// The LDS serves 256 bytes (16 chunk slots) per cycle: 16 lanes of a 16-byte
// read, 32 lanes of an 8-byte one.  K is read 16 bytes per lane down
// consecutive rows; a row starts at slot (row * DC) % 16, so XOR with
// (row / (16 / DC)) % DC gives any 16 consecutive rows 16 different slots.
// V is read 8 bytes per lane by the transposing read, a 64-byte run of each
// of four consecutive rows per half wave; XOR with (DC / 4) * (row % 4) puts
// the four runs in four different 64-byte slots.  (rocprofv3 reports no LDS
// bank conflicts with these.)
template <int DC> __device__ __forceinline__ int k_swz(int row) { return (row / (16 / DC)) & (DC - 1); }
template <int DC> __device__ __forceinline__ int v_swz(int row) { return (DC / 4) * (row & 3); }

// Query blocks (of 32 rows) per wave for a head dimension.
constexpr int query_blocks(int d) { return d == 64 ? 2 : 1; }

template <int D, int HPW, int QB>
__global__ __launch_bounds__(kThreads, (D == 64 && QB == 1) ? 3 : 2) void prefill_kernel(PrefillArgs a) {
  constexpr int BN = 64 / QB;            // keys per tile
  constexpr int KB = BN / 32;            // 32-key blocks per tile
  constexpr int NU = BN / 16;            // 16-key P.V steps per tile
  constexpr int RG = 4 / HPW;            // row groups per workgroup
  constexpr int WROWS = 32 * QB;         // query rows per wave
  constexpr int ROWS = WROWS * RG;
  constexpr int DC = D / 8;              // 16-byte chunks per key row
  constexpr int KT = BN * D;             // elements of one K or V tile
  constexpr int DMA = BN * DC / kThreads;   // 16-byte DMA slots per thread per tile
  constexpr bool kDeferPV = D == 64;        // P.V one tile behind (registers permitting)
  // Separate arrays per buffer: the compiler then sees that the copies into
  // one buffer never alias the reads of the other, and does not make those
  // reads wait for the copies in flight.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[KT], k_lds1[KT], v_lds0[KT], v_lds1[KT];

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
  const int seq = slot / a.n_qtiles;
  const int qtile = a.n_qtiles - 1 - slot % a.n_qtiles;
  const int start = a.cu_seqlens[seq];                 // first query token
  const int len = a.cu_seqlens[seq + 1] - start;       // queries of the sequence
  const int start_k = a.cu_seqlens_k[seq];             // first key token
  const int len_k = a.cu_seqlens_k[seq + 1] - start_k;
  // The queries are the last `len` of the sequence's len_k tokens (all of
  // them for plain prefill): query i sits at position off + i.  A chunk
  // longer than its keys breaks the interface's precondition; it is skipped
  // (its outputs are left unwritten) rather than read out of range.
  const int off = len_k - len;
  if (off < 0) return;
  const int q0 = qtile * ROWS;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int h = hg * HPW + (wave % HPW);
  const int g = (hg * HPW) / a.group;
  const int w_row0 = q0 + (wave / HPW) * WROWS;
  int qrow[QB], lim[QB];                 // positions inside the sequence; last visible key
  bool qvalid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = w_row0 + 32 * qb + lrow;
    qvalid[qb] = qrow[qb] < len;
    lim[qb] = a.causal ? min(off + qrow[qb], len_k - 1) : len_k - 1;
  }

  const int kv_end = a.causal ? min(off + q0 + ROWS, len_k) : len_k;
  const int ntiles = (kv_end + BN - 1) / BN;
  // leading tiles that no row of this workgroup needs masked
  const int nfull = min(a.causal ? (off + q0 + 1) / BN : ntiles, len_k / BN);

  // ---- Q^T fragments (B operand: column = query row, k = d) ---------------
  u32x4_t qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint16_t* qp = a.q + (int64_t)(start + (qvalid[qb] ? qrow[qb] : 0)) * a.q_st +
                         (int64_t)h * a.q_sh + 8 * lhalf;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4_t t = load16(qp + 16 * c);
      qf[qb][c] = qvalid[qb] ? t : u32x4_t{0, 0, 0, 0};
    }
  }

  // ---- K / V buffer resources over the visible keys -------------------------
  const int k_st2 = (int)(a.k_st * 2), v_st2 = (int)(a.v_st * 2);   // bytes per token
  const auto krs = make_rsrc(a.k + (int64_t)start_k * a.k_st + (int64_t)g * a.k_sh,
                             (kv_end - 1) * k_st2 + 2 * D);
  const auto vrs = make_rsrc(a.v + (int64_t)start_k * a.v_st + (int64_t)g * a.v_sh,
                             (kv_end - 1) * v_st2 + 2 * D);

  // DMA: thread t's i-th copy fills LDS slot (16 bytes) s = 64*(4i + wave) + lane
  // of a tile, i.e. key row s / DC, physical chunk s % DC.  K rows hold the
  // logical chunk (s % DC) ^ k_swz(row), V rows (s % DC) ^ v_swz(row).
  int k_goff[DMA], v_goff[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int s = 64 * (4 * i + wave) + lane, key = s / DC;
    k_goff[i] = key * k_st2 + ((s % DC) ^ k_swz<DC>(key)) * 16;
    v_goff[i] = key * v_st2 + ((s % DC) ^ v_swz<DC>(key)) * 16;
  }
  // Buffer numbers are compile-time constants (std::integral_constant).
  auto dma_k = [&](int kt, auto buf) {
    uint16_t* dst = (decltype(buf)::value ? k_lds1 : k_lds0) + wave * 512;
    const int off = kt * BN * k_st2;
#pragma unroll
    for (int i = 0; i < DMA; ++i) buffer_load16_lds(krs, dst + i * 2048, k_goff[i], off);
  };
  auto dma_v = [&](int kt, auto buf) {
    uint16_t* dst = (decltype(buf)::value ? v_lds1 : v_lds0) + wave * 512;
    const int off = kt * BN * v_st2;
#pragma unroll
    for (int i = 0; i < DMA; ++i) buffer_load16_lds(vrs, dst + i * 2048, v_goff[i], off);
  };

  // LDS read offsets (elements).  K (ds_read_b128): row kb*32 + lrow, logical
  // chunk 2c + lhalf.  V^T (transposing read): lane i of a 16-lane group
  // addresses key row 16u + 8t + 4*lhalf + (i >> 2), d = 32db + 16*((lane>>4)&1)
  // + 4*(i & 3).
  int k_roff[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) k_roff[c] = lrow * D + (((2 * c + lhalf) ^ k_swz<DC>(lrow)) * 8);
  int v_roff[D / 32];
  {
    const int i = lane & 15, gi = (lane >> 4) & 1;
    const int row = 4 * lhalf + (i >> 2);                 // key row within an 8-row group
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cl = 4 * db + 2 * gi + ((i & 3) >> 1);    // logical chunk for db
      v_roff[db] = row * D + ((cl ^ v_swz<DC>(row)) * 8) + 4 * (i & 1);
    }
  }
  // S^T = K Q^T for one tile: each K operand serves all query blocks
  auto qk = [&](auto buf, f32x16_t (&s)[QB][KB]) {
    const uint16_t* ks = decltype(buf)::value ? k_lds1 : k_lds0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16_t{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4_t kop =
            *reinterpret_cast<const u32x4_t*>(ks + k_roff[c] + kb * 32 * D);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_32x32x16(kop, qf[qb][c], s[qb][kb]);
      }
    }
  };

  // ---- running state, seeded with the sink ---------------------------------
  // m: the stabiliser of the exponentials, in log2 units (never below -FLT_MAX
  // so that differences stay finite); it starts at the sink's logit.  lsum:
  // this lane's share of the denominator of its query row (lanes l and l^32
  // hold the two halves of every key block); the sink's exp2(0) = 1 starts in
  // the lower half.
  const float sink = a.sinks[h];
  const float c2 = a.scale_log2;
  float m[QB], lsum[QB];
  f32x16_t acc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = fmaxf(sink * kLog2e, -__FLT_MAX__);
    lsum[qb] = (lhalf == 0 && sink != -INFINITY) ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[qb][db] = f32x16_t{};
  }

  f32x16_t sa[QB][KB], sb[QB][KB];

  // Causal / length mask of a tile's scores (tiles past nfull only).
  auto mask = [&](int jt, f32x16_t (&s)[QB][KB]) {
    const int key0 = jt * BN + 4 * lhalf;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key0 + kb * 32 + 8 * (i >> 2) + (i & 3) > lim[qb]) s[qb][kb][i] = -INFINITY;
  };

  // Weights of a tile under the current stabiliser: pf = bf16(exp2(s*c2 - m)),
  // already in the P.V operand layout, and ts = this lane's share of their
  // sum (the same bf16 values that enter P.V).  On the matrix pipe the P^T
  // operand of a 16-key step is read as the B operand of a 16x16x32 MFMA
  // (lane group q = l/16 supplies query (l%16) + 16(q%2), keys 8(q/2)..+7)
  // against a 0/1 matrix whose row m is 1 on the groups with q%2 = (m/4)%2:
  // every lane then receives the 16-key sum of its own query (half the matrix
  // cycles and a quarter of the registers of a ones row on 32x32x16).  Only
  // the lower half of the lanes keeps it, so that lanes l and l^32 still add
  // up to the row's sum.
  const u32x4_t ones16 = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1)
                             ? u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}
                             : u32x4_t{0u, 0u, 0u, 0u};
  auto weights = [&](f32x16_t (&s)[QB][KB], u32x4_t (&pf)[QB][NU], float (&ts)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4_t tm = {};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int kb = u >> 1, base = 8 * (u & 1);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(s[qb][kb][base + e], c2, -m[qb]));
        pf[qb][u][0] = pack_bf16x2(p[0], p[1]);
        pf[qb][u][1] = pack_bf16x2(p[2], p[3]);
        pf[qb][u][2] = pack_bf16x2(p[4], p[5]);
        pf[qb][u][3] = pack_bf16x2(p[6], p[7]);
        tm = mfma_16x16x32(ones16, pf[qb][u], tm);
      }
      ts[qb] = lhalf == 0 ? tm[0] : 0.f;
    }
  };

  // Moving the stabiliser: m becomes the running row max, O and the
  // denominator are rescaled to it, and the tile's weights are recomputed.
  auto restabilise = [&](f32x16_t (&s)[QB][KB], u32x4_t (&pf)[QB][NU], float (&ts)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
      const float m_new = fmaxf(m[qb], pair32_max(mx) * c2);
      const float alpha = fast_exp2(m[qb] - m_new);
      m[qb] = m_new;
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
    }
    weights(s, pf, ts);
  };

  // P.V of one tile from register operands.
  auto pv = [&](const u32x4_t (&pf)[QB][NU], const u32x4_t (&vf)[NU][D / 32]) {
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma_32x32x16(vf[u][db], pf[qb][u], acc[qb][db]);
  };
  // V^T operands of one tile, through the transposing LDS read.
  auto read_v = [&](auto buf, u32x4_t (&vf)[NU][D / 32]) {
    const uint16_t* vt = decltype(buf)::value ? v_lds1 : v_lds0;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vp = vt + v_roff[db] + 16 * u * D;
        const u32x2_t lo = lds_read_tr16(vp);
        const u32x2_t hi = lds_read_tr16(vp + 8 * D);
        vf[u][db] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
  };

  // One tile j.  With kDeferPV the matrix pipe runs QK^T of tile j+1 (into
  // s_nxt) and P.V of tile j-1 (operands already in registers) while the
  // vector ALU computes the exponentials of tile j -- independent streams
  // that overlap inside the wave; then the V^T operands of tile j are read
  // into registers for the next step.  Without it (head_dim 128, where those
  // operands would not fit in registers) P.V of tile j follows the
  // stabiliser check, its V^T operands read from LDS next to the MFMAs.
  // Last, tile j+1 is masked when it needs it.  `par` is j % 2 as a
  // compile-time constant.
  using PF = u32x4_t[QB][NU];
  using VF = u32x4_t[NU][D / 32];
  auto step = [&](auto par, int j, f32x16_t (&s_cur)[QB][KB], f32x16_t (&s_nxt)[QB][KB],
                  PF& pf_prev, VF& vf_prev, PF& pf_cur, VF& vf_cur) {
    constexpr int P = decltype(par)::value;
    const std::integral_constant<int, P> cur{};
    const std::integral_constant<int, 1 - P> nxt{};
    // copies of K(j+2) and V(j+1) run during this tile's math
    if (j + 2 < ntiles) dma_k(j + 2, cur);
    if (j + 1 < ntiles) dma_v(j + 1, nxt);
    qk(nxt, s_nxt);
    if constexpr (kDeferPV) pv(pf_prev, vf_prev);
    float ts[QB];
    weights(s_cur, pf_cur, ts);
    if constexpr (kDeferPV) read_v(cur, vf_cur);
    // The stabiliser moves only when a lane's tile weights sum past
    // kMaxTileSum (an overflow to inf included, and the NaN that 0 * inf gives
    // in the 0/1 matrix sum).  Until then every weight
    // stays below kMaxTileSum, O and the denominator share the same m, and
    // o = O / d is unchanged -- one wave-uniform branch per tile and no row
    // max.  A move rescales O after P.V of tile j-1 has entered it.
    bool big = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) big |= !(ts[qb] <= kMaxTileSum);
    if (__builtin_amdgcn_ballot_w64(big) != 0) restabilise(s_cur, pf_cur, ts);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] += ts[qb];
    if constexpr (!kDeferPV) {
      const uint16_t* vt = P ? v_lds1 : v_lds0;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t* vp = vt + v_roff[db] + 16 * u * D;
          const u32x2_t lo = lds_read_tr16(vp);
          const u32x2_t hi = lds_read_tr16(vp + 8 * D);
          const u32x4_t vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma_32x32x16(vf, pf_cur[qb][u], acc[qb][db]);
        }
    }
    if (j + 1 < ntiles && j + 1 >= nfull) mask(j + 1, s_nxt);
    wait_vmem();
    __syncthreads();
  };

  // ---- prologue: K(0), V(0), K(1) staged; S of tile 0 ---------------------------
  const std::integral_constant<int, 0> even{};
  const std::integral_constant<int, 1> odd{};
  dma_k(0, even);
  dma_v(0, even);
  if (ntiles > 1) dma_k(1, odd);
  wait_vmem();
  __syncthreads();
  qk(even, sa);
  if (nfull == 0) mask(0, sa);
  __syncthreads();          // K buffer 0 is refilled in iteration 0

  // ---- tiles, two per trip so the register sets swap roles --------------------
  // (pa, va) start as zeros: with kDeferPV the first step's P.V of "tile -1"
  // adds nothing.
  PF pa, pb;
  VF va, vb;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pa[qb][u] = u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) va[u][db] = u32x4_t{0, 0, 0, 0};
  }
  int j = 0;
  for (; j + 2 <= ntiles; j += 2) {
    step(even, j, sa, sb, pa, va, pb, vb);
    step(odd, j + 1, sb, sa, pb, vb, pa, va);
  }
  if (j < ntiles) {
    step(even, j, sa, sb, pa, va, pb, vb);
    if constexpr (kDeferPV) pv(pb, vb);
  } else {
    if constexpr (kDeferPV) pv(pa, va);
  }

  // ---- epilogue: normalise, round to bf16, store ----------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = pair32_sum(lsum[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qvalid[qb]) {
      uint16_t* op = a.o + (int64_t)(start + qrow[qb]) * a.o_st + (int64_t)h * a.o_sh + 4 * lhalf;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          u32x2_t w;
          w[0] = pack_bf16x2(acc[qb][db][4 * i4 + 0] * inv, acc[qb][db][4 * i4 + 1] * inv);
          w[1] = pack_bf16x2(acc[qb][db][4 * i4 + 2] * inv, acc[qb][db][4 * i4 + 3] * inv);
          *reinterpret_cast<u32x2_t*>(op + db * 32 + 8 * i4) = w;
        }
      if (a.lse != nullptr && lhalf == 0)
        a.lse[(int64_t)(start + qrow[qb]) * a.num_q_heads + h] =
            lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int hpw, int64_t nb, hipStream_t st) {
  constexpr int QB = query_blocks(D);
  const dim3 grid((unsigned)nb), block(kThreads);
  switch (hpw) {
    case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, QB>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, QB>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((prefill_kernel<D, 1, QB>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

}  // namespace sinkattn
