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
// decode_split_kernel: one workgroup of W = 1, 2 or 4 waves per (request b, KV
// head g, slice of 16*CB columns, chunk c).  A column is one (new token t, query head of g)
// pair: one new token per request for plain decode, q_len of them for the
// multi-token decode of speculative / MTP verification ("GPT-OSS on day 0",
// section "Internal inference engine"; "Hosting Qwen on Blackwell", section
// "Decoders"), where new token t -- already in the cache, whose last q_len
// tokens are the new ones -- sees the cache up to its own position.  The K/V
// of the chunk are read exactly once and serve every column.  The chunk is cut
// into 64-key sub-tiles; wave w takes sub-tiles w, w+W, w+2W, ... and runs its
// own pipeline with no workgroup barrier until the final merge:
//   * K of the next sub-tile is loaded HBM -> registers and V of the next
//     sub-tile is copied HBM -> LDS (buffer->LDS DMA into the wave's double
//     buffer) while the current sub-tile is computed; both streams are read
//     once, so they are loaded non-temporally;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 d straight
//     from the registers, B = Q^T of a block of 16 columns (padding columns
//     zero); each K and V^T operand feeds all CB column blocks, so a chunk is
//     read once for up to 16*CB columns;
//   * the softmax state is per lane (one column); row max and sum reduce
//     over the four 16-lane rows with permlane16/32 swaps; keys past a
//     column's position are masked in the last sub-tiles;
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//     accumulators, V^T from the row-major V tile via the transposing LDS read.
// At the end the W waves' states are merged through LDS (W > 1) and the chunk's
// (o / d, m, d) is written in fp32.  Only wave 0 of chunk 0 seeds the sink.
// W trades the merge across waves against parallelism inside a chunk: four
// waves per chunk for one light column block; one wave per chunk, writing its
// state directly, for heavier math when the chunks alone fill the SIMDs.
// Two cache forms beyond bf16 per-request slabs share the kernel: FP8 E4M3
// codes with a scale per KV head (converted exactly to bf16 in registers;
// V through the 8-bit transposing read), and pages behind a block table (a
// buffer resource per 16-key block).
// merge_rows_kernel (up to 16 chunks) and merge_kernel: log-sum-exp weighted
// sum of the chunk states, rounded to bf16 -- D / 4 lanes per (b, h) row, or
// one wave per row with lane = d.
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kThreads = 256;                 // merge kernel
constexpr int kSub = 64;                      // keys per sub-tile

// Chunk swizzle of the row-major V sub-tile (DC 16-byte chunks per row).  The
// LDS serves 16 chunk slots (256 bytes) per cycle, i.e. 32 lanes of a
// transposing 8-byte read: a 32-byte run of each of eight consecutive rows.
// A row starts at slot (row * DC) % 16; XOR with 2 * ((row / (16 / DC)) %
// (DC / 2)) gives the eight runs eight different 32-byte slots.
template <int DC> __device__ __forceinline__ int dv_swz(int row) {
  return 2 * ((row / (16 / DC)) & (DC / 2 - 1));
}
// The same for an FP8 (one byte per element) V sub-tile, read with the 8-bit
// transposing read: the 32 lanes of a half-wave address 16 rows x two 8-byte
// halves of one 16-byte chunk.  Rows hold 4 (D 64) or 8 (D 128) chunks, so
// rows 4 (2) apart share bank slots; the XOR gives the rows that meet in a
// half-wave different chunk slots (checked exhaustively on the host).
template <int D> __device__ __forceinline__ int v8_swz(int row) {
  if constexpr (D == 64) return ((row >> 2) + 2 * (row >> 4)) & 3;
  return ((row >> 1) & 3) | ((row >> 2) & 4);
}

// fp32 values of the final merge of W waves' states: m and l of every column,
// then o (none for a single wave, which writes its state directly).
template <int D, int CB, int W>
constexpr int decode_merge_floats() {
  return W == 1 ? 0 : 2 * W * 16 * CB + W * D * 16 * CB;
}
// 16-bit LDS elements of one V sub-tile (bf16, or FP8 codes two to an element).
template <int D, bool F8> constexpr int v_tile_elems() { return F8 ? kSub * D / 2 : kSub * D; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// LDS of one decode workgroup (16-bit elements): two arrays of the waves' V
// sub-tiles (even and odd sub-tiles), the first of them later reused for the
// merge, and with one wave for the staged state (two column blocks of fp32 o
// per array).  Two arrays rather than one with two halves: the compiler can
// then see that a copy into one never aliases reads of the other, and does not
// make the reads of sub-tile st wait for the copy of st + 1.
template <int D, int CB, int W, bool F8>
constexpr int decode_lds0_elems() {
  return cmax(cmax(W * v_tile_elems<D, F8>(), 2 * decode_merge_floats<D, CB, W>()),
              W == 1 ? 2 * (CB < 2 ? CB : 2) * 16 * D : 0);
}
template <int D, int CB, int W, bool F8>
constexpr int decode_lds1_elems() {
  return cmax(W * v_tile_elems<D, F8>(), W == 1 && CB > 2 ? 2 * (CB - 2) * 16 * D : 0);
}

// Chunk states that another workgroup merges in the same launch cross L2
// caches (one per XCD): they are written and read with device-scope accesses
// (sc1), which are coherent across the XCDs without a cache-wide writeback
// or invalidate.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order of the work units (request b, KV head g, chunk c, column slice hs).
// Workgroups go round-robin to the 8 XCDs, each with its own L2 and address
// translation caches.  Split decode runs request-major, (b, c, g, hs) with hs
// fastest: with one slice per unit an XCD then takes one KV head, and its
// workgroups in flight stream the contiguous ranges of that head in a few
// requests rather than one chunk of every request -- 1-8% faster than
// chunk-major on 1 GiB caches, 4 GiB caches and ragged batches, most where the
// batch is large or ragged.  The one-launch decode (counters set) keeps the
// chunk-major order (c, b, g, hs): the workgroups that merge then come in the
// launch's last wave, where the merges fill the tail (6% faster there on
// uniform 64 x 8192 contexts).
__device__ __forceinline__ void unit_coords(const DecodeArgs& a, int unit, int& b, int& g, int& c,
                                            int& hs) {
  hs = unit % a.head_slices;
  unit /= a.head_slices;
  if (a.counters == nullptr) {
    g = unit % a.num_kv_heads;
    unit /= a.num_kv_heads;
    c = unit % a.num_splits;
    b = unit / a.num_splits;
  } else {
    g = unit % a.num_kv_heads;
    unit /= a.num_kv_heads;
    b = unit % a.batch;
    c = unit / a.batch;
  }
}

// One work unit: chunk c of request b, KV head g, column slice hs, on W waves.
// F8: the caches hold FP8 E4M3 codes with a dequantization scale per KV head;
// the codes convert exactly to bf16 for the MFMAs, k_scale joins the softmax
// scale and v_scale the final division by d.
// PG: the caches are pages [num_pages, Hkv, page_size, D] reached through a
// block table (page_size a power of two >= 16, so a 16-key block never
// straddles pages): each 16-key block gets its own buffer resource.
template <int D, int CB, int W, bool F8, bool PG>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, int unit, uint16_t* v_lds0,
                                            uint16_t* v_lds1) {
  constexpr int DC = D / 8;                  // 16-byte chunks per bf16 row
  constexpr int RB = F8 ? D : 2 * D;         // bytes per cached row
  constexpr int RC = RB / 16;                // 16-byte chunks per cached row
  constexpr int TILE = v_tile_elems<D, F8>();
  constexpr int NDMA = kSub * RB / 1024;     // DMA instructions per V sub-tile
  constexpr int NCC = D / 32;                // 32-d contraction chunks of QK^T
  constexpr int NKL = F8 ? D / 64 : NCC;     // 16-byte K loads per lane and 16-key block
  constexpr int NC = 16 * CB;                // columns of a workgroup
  constexpr int kMergeFloats = decode_merge_floats<D, CB, W>();
  constexpr int kLds0Elems = decode_lds0_elems<D, CB, W, F8>();
  constexpr int kBlock = 64 * W;

  int b, g, c, hs;
  unit_coords(a, unit, b, g, c, hs);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;           // column of each 16-column block this lane serves
  const int lgrp = lane >> 4;          // 16-lane row group 0..3
  const int x0 = hs * NC;              // first column of the workgroup
  const int nx = min(NC, a.ncols - x0);

  const int len = a.seq_lens[b];
  const int lo = c * a.split_size;
  const int n = max(min(a.split_size, len - lo), 0);    // keys of this chunk
  const int n_sub = (n + kSub - 1) / kSub;
  // keys of this chunk visible to every column
  const int n_all = min(n, len - (a.q_len - 1) - lo);
  // row of column x in the partial outputs
  auto out_row = [&](int x) {
    return (((int64_t)b * a.q_len + x / a.group) * a.num_q_heads + g * a.group + x % a.group) *
               a.num_splits + c;
  };
  // state stores: device scope when a workgroup of this launch merges them
  const bool dev_scope = a.counters != nullptr;
  auto put = [&](float* p, float v) {
    if (dev_scope) store_dev(p, v); else *p = v;
  };
  auto put_nt = [&](float* p, float v) {
    if (dev_scope) store_dev(p, v); else store_nt(p, v);
  };

  // A chunk past the request's end without the sink (ragged batches have many)
  // has the state (o, m, d) = (0, -inf, 0): write it and leave.
  // (In one launch the merge stops at the request's last chunk with keys, so
  // there such chunks write nothing.)
  if (n == 0 && c != 0) {
    if (dev_scope || a.skip_empty) return;
    for (int item = tid; item < nx * D; item += kBlock) {
      const int64_t row = out_row(x0 + item / D);
      const int d = item % D;
      put(a.part_o + row * D + d, 0.f);
      if (d == 0) {
        put(a.part_m + row, -INFINITY);
        put(a.part_d + row, 0.f);
      }
    }
    return;
  }

  // Per column block: Q^T fragments (column = (new token, head), k = d), the
  // keys of the run the lane's column sees, and the softmax state.  The
  // sink seeds wave 0 of chunk 0 only, counted once (row group 0).
  const bool seeded = (c == 0) && (wave == 0);
  u32x4_t qf[CB][NCC];
  int n_lane[CB];
  float m[CB], l[CB];
  f32x4_t acc[CB][D / 16];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const bool valid = cb * 16 + col < nx;
    const int x = x0 + (valid ? cb * 16 + col : 0);
    const int tq = x / a.group;        // new token of the column
    const int h = g * a.group + x % a.group;
    n_lane[cb] = min(n, len - (a.q_len - 1 - tq) - lo);
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)tq * a.q_st + (int64_t)h * a.q_sh;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      // contraction chunk cc, lane row group lgrp: d = 32cc + 8lgrp .. +7; with
      // FP8 K (16 codes per lane load): d = 64(cc/2) + 16lgrp + 8(cc%2) .. +7
      const int d0 = F8 ? 64 * (cc >> 1) + 16 * lgrp + 8 * (cc & 1) : 32 * cc + 8 * lgrp;
      const u32x4_t t = load16(qp + d0);
      qf[cb][cc] = valid ? t : u32x4_t{0, 0, 0, 0};
    }
    const float sink = valid ? a.sinks[h] : -INFINITY;
    m[cb] = seeded ? fmaxf(sink * kLog2e, -__FLT_MAX__) : -__FLT_MAX__;
    l[cb] = (seeded && lgrp == 0 && sink != -INFINITY) ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[cb][db] = f32x4_t{};
  }

  // softmax scale (log2 units) of the raw dot products, and the factor of o
  const float qk_scale = F8 ? a.scale_log2 * a.k_scale[g] : a.scale_log2;
  const float out_scale = F8 ? a.v_scale[g] : 1.f;

  // K / V of this chunk through buffer resources (loads past its end read 0):
  // one over the chunk for contiguous caches, one per 16-key block for pages
  constexpr int EB = F8 ? 1 : 2;             // bytes per cached element
  const int stb = (int)(a.kv_st * EB);       // bytes per cached token
  const int64_t base = ((int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh + (int64_t)lo * a.kv_st) * EB;
  const int nbytes = n > 0 ? (n - 1) * stb + RB : 0;
  const auto krs = make_rsrc(static_cast<const char*>(a.k_cache) + (PG ? 0 : base), PG ? 0 : nbytes);
  const auto vrs = make_rsrc(static_cast<const char*>(a.v_cache) + (PG ? 0 : base), PG ? 0 : nbytes);
  // pages: the chunk's block-table entries, lane l holding entry l + 64r past
  // its first page (at most 256 entries, checked on the host)
  int pidx[4] = {0, 0, 0, 0};
  int first_page = 0;
  if constexpr (PG) {
    first_page = lo >> a.page_shift;
    if (n > 0) {
      const int last_page = (lo + n - 1) >> a.page_shift;
      const int32_t* bt = a.block_tables + (int64_t)b * a.bt_stride;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = first_page + lane + 64 * r;
        pidx[r] = e <= last_page ? bt[e] : 0;
      }
    }
  }
  // Buffer resource of the 16-key block starting key16 keys into the chunk.
  auto block_rsrc = [&](const void* cache, int key16) {
    const int kabs = lo + key16;
    const int e = __builtin_amdgcn_readfirstlane((kabs >> a.page_shift) - first_page);
    int page;
    switch (e >> 6) {
      case 0: page = __builtin_amdgcn_readlane(pidx[0], e & 63); break;
      case 1: page = __builtin_amdgcn_readlane(pidx[1], e & 63); break;
      case 2: page = __builtin_amdgcn_readlane(pidx[2], e & 63); break;
      default: page = __builtin_amdgcn_readlane(pidx[3], e & 63); break;
    }
    const int slot = kabs & ((1 << a.page_shift) - 1);
    const int valid = min(16, len - kabs);
    const int64_t off = ((int64_t)page * a.kv_sp + (int64_t)g * a.kv_sh + (int64_t)slot * a.kv_st) * EB;
    return make_rsrc(static_cast<const char*>(cache) + off, valid > 0 ? (valid - 1) * stb + RB : 0);
  };

  // K fragment kb (16 keys): lane holds key kb*16 + col; bf16: load cc is
  // d = 32cc + 8lgrp .. +7; FP8: load i is d = 64i + 16lgrp .. +15
  int k_off[NKL];
#pragma unroll
  for (int i = 0; i < NKL; ++i) k_off[i] = col * stb + (F8 ? 64 * i + 16 * lgrp : (32 * i + 8 * lgrp) * 2);
  // V DMA: lane fills slot 64*i + lane = (row, physical chunk) of the sub-tile
  int v_goff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int s = 64 * i + lane, row = s / RC;
    v_goff[i] = row * stb + ((s % RC) ^ (F8 ? v8_swz<D>(row) : dv_swz<DC>(row))) * 16;
  }
  // V^T transposing reads (byte offsets in the sub-tile).  bf16: row
  // 32j + 16t + 4*lgrp + (col >> 2), d = 16*db + 4*(col & 3).  FP8: lanes
  // 2e, 2e+1 of row group lgrp address key 4lgrp + e (e < 4) or
  // 16 + 4lgrp + e - 4 and the two 8-byte halves of d 16db .. +15, so that
  // lane i receives d = 16db + i of those eight keys -- the keys and order of
  // the P^T operand built from the S^T accumulators.
  int v_roff[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    if constexpr (F8) {
      const int e = col >> 1;
      const int row = e < 4 ? 4 * lgrp + e : 16 + 4 * lgrp + e - 4;
      v_roff[db] = row * RB + 16 * (db ^ v8_swz<D>(row)) + 8 * (col & 1);
    } else {
      const int row = 4 * lgrp + (col >> 2);
      const int cl = 2 * db + ((col & 3) >> 1);
      v_roff[db] = row * RB + ((cl ^ dv_swz<DC>(row)) * 16) + 8 * (col & 1);
    }
  }

  auto load_k = [&](int st, u32x4_t (&kf)[4][NKL]) {
    const int off = st * kSub * stb;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if constexpr (PG) {
        const auto rs = block_rsrc(a.k_cache, st * kSub + 16 * kb);
#pragma unroll
        for (int i = 0; i < NKL; ++i) kf[kb][i] = buffer_load16<kNonTemporal>(rs, k_off[i]);
      } else {
#pragma unroll
        for (int i = 0; i < NKL; ++i) kf[kb][i] = buffer_load16<kNonTemporal>(krs, k_off[i] + kb * 16 * stb + off);
      }
    }
  };
  // Buffer numbers are compile-time constants (std::integral_constant).
  auto dma_v = [&](int st, auto buf) {
    const int off = st * kSub * stb;
    uint16_t* dst = (decltype(buf)::value ? v_lds1 : v_lds0) + wave * TILE;
    if constexpr (PG) {
      constexpr int RPI = 1024 / RB;         // rows per copy instruction: within one 16-key block
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const auto rs = block_rsrc(a.v_cache, st * kSub + 16 * kb);
#pragma unroll
        for (int i = kb * 16 / RPI; i < (kb + 1) * 16 / RPI; ++i)
          buffer_load16_lds<kNonTemporal>(rs, dst + i * 512, v_goff[i] - 16 * kb * stb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) buffer_load16_lds<kNonTemporal>(vrs, dst + i * 512, v_goff[i] + off);
    }
  };
  // One 64-key sub-tile: every K operand and every V^T operand feeds the CB
  // column blocks' MFMAs.
  auto compute = [&](int st, auto buf, const u32x4_t (&kf)[4][NKL]) {
    u32x4_t kop[4][NCC];             // K operands (FP8 codes converted to bf16)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        if constexpr (F8) {
          const u32x4_t raw = kf[kb][cc >> 1];
          kop[kb][cc] = fp8x8_to_bf16x8(raw[2 * (cc & 1)], raw[2 * (cc & 1) + 1]);
        } else {
          kop[kb][cc] = kf[kb][cc];
        }
      }
    f32x4_t s[CB][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        s[cb][kb] = f32x4_t{};
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) s[cb][kb] = mfma_16x16x32(kop[kb][cc], qf[cb][cc], s[cb][kb]);
      }
    const int k0 = st * kSub;
    if (k0 + kSub > n_all) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + kb * 16 + 4 * lgrp + i >= n_lane[cb]) s[cb][kb][i] = -INFINITY;
    }
    u32x4_t pf[CB][2];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      f32x4_t (&sc)[4] = s[cb];
      float mx = max3f(sc[0][0], sc[0][1], sc[0][2]);
      mx = max3f(mx, sc[0][3], sc[1][0]);
      mx = max3f(mx, sc[1][1], sc[1][2]);
      mx = max3f(mx, sc[1][3], sc[2][0]);
      mx = max3f(mx, sc[2][1], sc[2][2]);
      mx = max3f(mx, sc[2][3], sc[3][0]);
      mx = max3f(mx, sc[3][1], sc[3][2]);
      mx = fmaxf(mx, sc[3][3]);
      mx = pair32_max(pair16_max(mx));
      const float m_new = fmaxf(m[cb], mx * qk_scale);
      const float alpha = fast_exp2(m[cb] - m_new);
      m[cb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sc[kb][i], qk_scale, -m_new));
          sc[kb][i] = p;
          rs += p;
        }
      l[cb] = l[cb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[cb][db][i] *= alpha;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        pf[cb][j][0] = pack_bf16x2(sc[2 * j][0], sc[2 * j][1]);
        pf[cb][j][1] = pack_bf16x2(sc[2 * j][2], sc[2 * j][3]);
        pf[cb][j][2] = pack_bf16x2(sc[2 * j + 1][0], sc[2 * j + 1][1]);
        pf[cb][j][3] = pack_bf16x2(sc[2 * j + 1][2], sc[2 * j + 1][3]);
      }
    }
    const char* vt = reinterpret_cast<const char*>((decltype(buf)::value ? v_lds1 : v_lds0) + wave * TILE);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const char* vp = vt + v_roff[db] + 32 * j * RB;
        u32x4_t vf;
        if constexpr (F8) {
          const u32x2_t v = lds_read_tr8(vp);
          vf = fp8x8_to_bf16x8(v[0], v[1]);
        } else {
          const u32x2_t v0 = lds_read_tr16(vp);
          const u32x2_t v1 = lds_read_tr16(vp + 16 * RB);
          vf = u32x4_t{v0[0], v0[1], v1[0], v1[1]};
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb][db] = mfma_16x16x32(vf, pf[cb][j], acc[cb][db]);
      }
    }
  };

  // ---- per-wave pipeline over sub-tiles wave, wave+W, ... --------------------
  // At the top of each pass this wave's copies for sub-tile st are complete;
  // the copies for st + W are then issued and run during st's math.  Two
  // passes per loop trip so the K register sets swap roles without copies.
  const std::integral_constant<int, 0> even{};
  const std::integral_constant<int, 1> odd{};
  u32x4_t ka[4][NKL], kb2[4][NKL];
  int st = wave;
  if (st < n_sub) {
    load_k(st, ka);
    dma_v(st, even);
  }
  auto pass = [&](auto buf, const u32x4_t (&kcur)[4][NKL], u32x4_t (&knext)[4][NKL]) {
    wait_vmem();
    if (st + W < n_sub) {
      load_k(st + W, knext);
      dma_v(st + W, std::integral_constant<int, 1 - decltype(buf)::value>{});
    }
    compute(st, buf, kcur);
    st += W;
  };
  while (st < n_sub) {
    pass(even, ka, kb2);
    if (st >= n_sub) break;
    pass(odd, kb2, ka);
  }

  if constexpr (W == 1) {
    // ---- one wave: its state is the chunk's ---------------------------------
    // Streamed out (non-temporal): as plain stores under the saturating read
    // stream they were acknowledged so late that they held up the waves'
    // later waits (q_len 4: 12% slower).
    // o / d of every column goes through LDS ([column][d] fp32, 16-byte
    // chunks XOR-swizzled by the column; the V buffers are free now) so that
    // part_o is written in whole rows.  Each V array holds two column blocks.
    static_assert(2 * (CB < 2 ? CB : 2) * 16 * D <= kLds0Elems, "staged o fits the first array");
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const float lt = pair32_sum(pair16_sum(l[cb]));
      const float inv = lt > 0.f ? out_scale / lt : 0.f;
      float* stg = reinterpret_cast<float*>(cb < 2 ? v_lds0 : v_lds1) + (cb & 1) * 16 * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4_t*>(stg + col * D + 4 * ((4 * db + lgrp) ^ col)) = acc[cb][db] * inv;
      if (lgrp == 0 && cb * 16 + col < nx) {
        const int64_t row = out_row(x0 + cb * 16 + col);
        put_nt(a.part_m + row, lt > 0.f ? m[cb] * kLn2 : -INFINITY);
        put_nt(a.part_d + row, lt);
      }
    }
    __syncthreads();
    for (int item = lane; item < nx * (D / 4); item += 64) {
      const int xl = item / (D / 4), d4 = item % (D / 4);
      const int cb = xl / 16, xc = xl % 16;
      const float* stg = reinterpret_cast<const float*>(cb < 2 ? v_lds0 : v_lds1) + (cb & 1) * 16 * D;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + xc * D + 4 * (d4 ^ xc));
      float* op = a.part_o + out_row(x0 + xl) * D + 4 * d4;
#pragma unroll
      for (int i = 0; i < 4; ++i) put_nt(op + i, v[i]);
    }
  } else {
    // ---- merge the W waves' states through LDS ------------------------------
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) l[cb] = pair32_sum(pair16_sum(l[cb]));
    __syncthreads();                  // every wave is done with its V buffers
    static_assert(2 * kMergeFloats <= kLds0Elems, "merge buffers must fit in LDS");
    float* red = reinterpret_cast<float*>(v_lds0);
    float* red_m = red;               // [W][NC]
    float* red_l = red + W * NC;      // [W][NC]
    float* red_o = red + 2 * W * NC;  // [W][NC][D], 16-byte chunks XOR-swizzled by column
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int xl = cb * 16 + col;
      if (lgrp == 0) {
        red_m[wave * NC + xl] = m[cb];
        red_l[wave * NC + xl] = l[cb];
      }
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        *reinterpret_cast<f32x4_t*>(red_o + (wave * NC + xl) * D + 4 * ((4 * db + lgrp) ^ col)) =
            acc[cb][db];
    }
    __syncthreads();

    // four consecutive d of one column per thread: whole rows of part_o
    for (int item = tid; item < nx * (D / 4); item += kBlock) {
      const int xl = item / (D / 4), c4 = item % (D / 4);
      float M = -__FLT_MAX__;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, red_m[w * NC + xl]);
      float wsum = 0.f;
      f32x4_t o = {};
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = fast_exp2(red_m[w * NC + xl] - M);
        wsum += red_l[w * NC + xl] * f;
        o += *reinterpret_cast<const f32x4_t*>(red_o + (w * NC + xl) * D + 4 * (c4 ^ (xl & 15))) * f;
      }
      const int64_t row = out_row(x0 + xl);
      const float inv = wsum > 0.f ? out_scale / wsum : 0.f;
      float* op = a.part_o + row * D + 4 * c4;
#pragma unroll
      for (int i = 0; i < 4; ++i) put(op + i, o[i] * inv);
      if (c4 == 0) {
        put(a.part_m + row, wsum > 0.f ? M * kLn2 : -INFINITY);
        put(a.part_d + row, wsum);
      }
    }
  }
}

// Wave-wide reductions (64 lanes) for the merge.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per (b, h) row.  Every load of the row is issued up front: lane c
// reads chunk c's (m, d), and each lane reads its d column of the first
// kMergeRegs chunks' outputs; the weights are then broadcast lane to lane.
constexpr int kMergeRegs = 16;

// Merge of one (b, h) row's first ns chunk states by one wave (lane = d), in
// two steps: merge_load issues the loads of the first kMergeRegs chunks' o
// and the first 64 chunks' m and d (one round trip), merge_finish combines
// them (and reads any further chunks itself).  DEV: device-scope loads
// (states written by this launch).
template <int D>
struct MergeIn {
  float ov[kMergeRegs][D / 64];
  float m0, d0;
};

template <int D, bool DEV>
__device__ __forceinline__ float merge_ld(const float* p) {
  return DEV ? load_dev(p) : *p;
}

template <int D, bool DEV>
__device__ __forceinline__ void merge_load(const MergeArgs& a, int row, int lane, int ns,
                                           MergeIn<D>& in) {
  constexpr int DL = D / 64;                 // d values per lane
  const int64_t first = (int64_t)row * a.num_splits;
  const float* po = a.part_o + first * D;
#pragma unroll
  for (int c = 0; c < kMergeRegs; ++c)
#pragma unroll
    for (int j = 0; j < DL; ++j)
      in.ov[c][j] = c < ns ? merge_ld<D, DEV>(po + c * D + lane + 64 * j) : 0.f;
  in.m0 = lane < ns ? merge_ld<D, DEV>(a.part_m + first + lane) : -INFINITY;
  in.d0 = lane < ns ? merge_ld<D, DEV>(a.part_d + first + lane) : 0.f;
}

template <int D, bool DEV>
__device__ __forceinline__ void merge_finish(const MergeArgs& a, int row, int lane, int ns,
                                             const MergeIn<D>& in) {
  auto ld = [](const float* p) { return merge_ld<D, DEV>(p); };
  constexpr int DL = D / 64;
  const int64_t first = (int64_t)row * a.num_splits;
  const float* pm = a.part_m + first;
  const float* pd = a.part_d + first;
  const float* po = a.part_o + first * D;
  float M = fmaxf(-INFINITY, wave_max(in.m0));
  for (int c0 = 64; c0 < ns; c0 += 64) {
    const int c = c0 + lane;
    M = fmaxf(M, wave_max(c < ns ? ld(pm + c) : -INFINITY));
  }
  float W = 0.f;
  float acc[DL] = {};
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < ns; c0 += 64) {
      const int c = c0 + lane;
      const float mc = c0 == 0 ? in.m0 : (c < ns ? ld(pm + c) : -INFINITY);
      const float dc = c0 == 0 ? in.d0 : (c < ns ? ld(pd + c) : 0.f);
      const float w = mc == -INFINITY ? 0.f : dc * fast_exp2((mc - M) * kLog2e);
      W += wave_sum(w);
      const int cn = min(64, ns - c0);
      auto wt = [&](int k) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
      };
      int k = 0;
      if (c0 == 0) {
#pragma unroll
        for (int r = 0; r < kMergeRegs; ++r)
          if (r < cn) {
            const float wk = wt(r);
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] += wk * in.ov[r][j];
          }
        k = kMergeRegs;
      }
      // further chunks kMergeRegs at a time: their loads go out together
      for (; k < cn; k += kMergeRegs) {
        float ot[kMergeRegs][DL];
#pragma unroll
        for (int r = 0; r < kMergeRegs; ++r)
#pragma unroll
          for (int j = 0; j < DL; ++j)
            ot[r][j] = k + r < cn ? ld(po + (int64_t)(c0 + k + r) * D + lane + 64 * j) : 0.f;
#pragma unroll
        for (int r = 0; r < kMergeRegs; ++r)
          if (k + r < cn) {
            const float wk = wt(k + r);
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] += wk * ot[r][j];
          }
      }
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  // row = (b * q_len + t) * num_q_heads + h
  const int bt = row / a.num_q_heads, h = row % a.num_q_heads;
  uint16_t* op = a.o + (int64_t)(bt / a.q_len) * a.o_sb + (int64_t)(bt % a.q_len) * a.o_st +
                 (int64_t)h * a.o_sh;
#pragma unroll
  for (int j = 0; j < DL; ++j) {
    const __bf16 v = (__bf16)(acc[j] * inv);
    op[lane + 64 * j] = __builtin_bit_cast(uint16_t, v);
  }
  if (a.lse != nullptr && lane == 0) a.lse[row] = W > 0.f ? M + __logf(W) : -INFINITY;
}

// Fused merge: once its chunk state is written (device-scope stores, all
// acknowledged), a workgroup counts itself in for its (b, KV head, column
// slice); the one that arrives last -- every other chunk's state is then
// complete -- reads them with device-scope loads, merges the slice's rows with
// the same per-row code as merge_kernel and resets the counter for the next
// launch.  Only chunk 0 and the chunks holding keys take part: the others'
// state (0, -inf, 0) adds nothing to a merge.
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

template <int D, int CB, int W>
__device__ __forceinline__ void decode_merge_if_last(const DecodeArgs& a, int unit) {
  constexpr int NC = 16 * CB;
  __shared__ int is_last;
  int b, g, c, hs;
  unit_coords(a, unit, b, g, c, hs);
  const int len = a.seq_lens[b];
  const int live = (int)max((int64_t)1, min((int64_t)a.num_splits,
                                              ((int64_t)len + a.split_size - 1) / a.split_size));
  if (c >= live) return;
  int32_t* counter = a.counters + ((int64_t)b * a.num_kv_heads + g) * a.head_slices + hs;
  // The first barrier's fence keeps the compiler from moving the state stores
  // below the wait; the wait makes each wave's device-scope stores complete;
  // the second barrier makes them all complete before thread 0 counts in.
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(counter, 1) == live - 1;
  __syncthreads();
  if (!is_last) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int x0 = hs * NC, nx = min(NC, a.ncols - x0);
  for (int xl = wave; xl < nx; xl += W) {
    const int x = x0 + xl;
    const int row = ((b * a.q_len + x / a.group) * a.num_q_heads) + g * a.group + x % a.group;
    MergeIn<D> in;
    merge_load<D, true>(a.merge, row, lane, live, in);
    merge_finish<D, true>(a.merge, row, lane, live, in);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per unit.  head_dim 64 with up to 2 column blocks runs 2 waves
// per SIMD (16 KB of LDS per wave); wider blocks and head_dim 128 need the
// registers of 1 wave per SIMD.
template <int D, int CB, int W, bool F8, bool PG>
__global__ __launch_bounds__(64 * W, (D == 64 && CB <= 2) ? 2 : 1) void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[decode_lds0_elems<D, CB, W, F8>()];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[decode_lds1_elems<D, CB, W, F8>()];
  decode_unit<D, CB, W, F8, PG>(a, blockIdx.x, v_lds0, v_lds1);
  if (a.counters != nullptr) decode_merge_if_last<D, CB, W>(a, blockIdx.x);
}

// The merge of split decode into at most kMergeBlock chunks: D / 4 lanes per
// row (four d each, 16-byte loads), 64 / (D / 4) rows per wave.  Each lane
// loads its row's (m, d) of every chunk itself (the lanes of a row share those
// addresses), so the merge needs no lane exchange and all its loads go out at
// once.  The sums run in merge_finish's order -- o chunk by chunk, sum_c w_c
// as the pairwise tree that its butterfly reduction forms -- so both merges
// give the same bits.  Needs part_o 16-byte aligned.  (Against merge_kernel:
// 64 x 64 rows of 8 chunks 3.5 vs 4.0 us, 16384 rows 7.7 vs 10.8 us; past 16
// chunks, in blocks of 16, it was slower and merge_kernel stays.)
constexpr int kMergeBlock = 16;

// Chunks of row (b * q_len + t) * num_q_heads + h to merge: all, or with the
// request lengths given, those holding keys (chunk 0 at least) -- the split
// decode then wrote no state for the others, whose (0, -inf, 0) adds only
// exact zeros to a merge.
__device__ __forceinline__ int merge_chunks(const MergeArgs& a, int row) {
  if (a.seq_lens == nullptr) return a.num_splits;
  const int64_t len = a.seq_lens[row / (a.q_len * a.num_q_heads)];
  return (int)max((int64_t)1, min((int64_t)a.num_splits, (len + a.split_size - 1) / a.split_size));
}

__device__ __forceinline__ float tree_sum16(const float (&w)[kMergeBlock]) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = w[2 * i] + w[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return (t[0] + t[1]) + (t[2] + t[3]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_rows_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;                  // lanes per row
  constexpr int RPW = 64 / LPR;               // rows per wave
  constexpr int NB = kMergeBlock;
  const int lane = threadIdx.x & 63;
  const int row = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * RPW + lane / LPR;
  if (row >= a.rows) return;
  const int d0 = 4 * (lane % LPR);
  const int ns = merge_chunks(a, row);
  const int64_t first = (int64_t)row * a.num_splits;
  const float* pm = a.part_m + first;
  const float* pd = a.part_d + first;
  const float* po = a.part_o + first * D + d0;
  // loads clamped to the last chunk (always issued, no branch around them),
  // chunks past it given m = -inf
  float mv[NB], dv[NB], w[NB];
  f32x4_t ov[NB];
  auto load_block = [&] {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int ci = min(i, ns - 1);
      mv[i] = pm[ci];
      dv[i] = pd[ci];
      ov[i] = *reinterpret_cast<const f32x4_t*>(po + (int64_t)ci * D);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (i >= ns) mv[i] = -INFINITY;
  };
  // the weights and o, chunk by chunk; returns the tree sum of the weights
  // (the chunks past ns add exact zeros to it)
  auto combine = [&](float M, f32x4_t& acc) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      w[i] = mv[i] == -INFINITY ? 0.f : dv[i] * fast_exp2((mv[i] - M) * kLog2e);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (i < ns) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += w[i] * ov[i][j];
      }
    return tree_sum16(w);
  };
  // one round trip: all of the row's chunks in registers
  load_block();
  float M = -INFINITY, W = 0.f;
  f32x4_t acc = {};
#pragma unroll
  for (int i = 0; i < NB; ++i) M = fmaxf(M, mv[i]);
  if (M != -INFINITY) W = combine(M, acc);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int bt = row / a.num_q_heads, h = row % a.num_q_heads;
  uint16_t* op = a.o + (int64_t)(bt / a.q_len) * a.o_sb + (int64_t)(bt % a.q_len) * a.o_st +
                 (int64_t)h * a.o_sh + d0;
  uint32_t pk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const __bf16 lo = (__bf16)(acc[2 * j] * inv), hi = (__bf16)(acc[2 * j + 1] * inv);
    pk[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  *reinterpret_cast<uint2*>(op) = make_uint2(pk[0], pk[1]);
  if (a.lse != nullptr && d0 == 0) a.lse[row] = W > 0.f ? M + __logf(W) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int ns = merge_chunks(a, row);
  MergeIn<D> in;
  merge_load<D, false>(a, row, threadIdx.x & 63, ns, in);
  merge_finish<D, false>(a, row, threadIdx.x & 63, ns, in);
}

}  // namespace

// Scratch of the no-allocation decode entry point: the chunk states (o, m, d)
// of one call, carved from this array.  Each GPU the library runs on holds its
// own copy (kDecodeScratchFloats fp32, 128 MiB) until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[kDecodeScratchFloats];

hipError_t decode_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

int decode_column_blocks(int ncols, int head_dim) {
  const int need = (ncols + 15) / 16;
  const int most = head_dim == 64 ? 4 : 2;   // registers
  return need <= 1 ? 1 : (need <= 2 ? 2 : most);
}

constexpr int kComputeUnits = 256;             // MI355X

int decode_waves_per_unit(int64_t num_units, int head_dim, int column_blocks) {
  // head_dim 64 with one column block: little math per sub-tile, and four
  // waves per chunk shorten each chunk's critical path, which ragged batches
  // need (B = 8 / 32 contexts U[1024, 32768]: 9% / 5% faster than a wave per
  // chunk; uniform 64 x 8192 contexts equal).  Heavier math (more column
  // blocks, head_dim 128) makes the waves sharing a chunk wait for one another
  // at the merge -- at 1 wave per SIMD that stalls the CU -- so there each wave
  // takes a chunk of its own (q_len 4 / 8 and head_dim 128: 15% / 80% / 8%
  // faster), unless that leaves SIMDs idle.
  if (head_dim == 64 && column_blocks == 1) return 4;
  const int64_t simds = (int64_t)kComputeUnits * 4;
  return num_units >= simds ? 1 : (2 * num_units >= simds ? 2 : 4);
}

int decode_split_size(int64_t column_units, int max_len, bool uniform, int head_dim, int cus) {
  // Measured (d 64, split + length-aware merge, graph replay, inputs rotated
  // past the Infinity Cache):
  //  * equal contexts want long chunks -- fewer chunk states to write and
  //    merge, longer runs of one head per wave: 64 x 8192 tokens 171 / 163 /
  //    160 / 158 us with 1024 / 2048 / 4096 / 8192-token chunks, 4 new tokens
  //    per request 203 / 181 / 168 / 169 us, FP8 codes 97 / 93 / 96 / 85 us,
  //    16 x 32768 177 / 164 / 161 / 159 us -- as long as the chunks leave a
  //    unit for every fourth SIMD;
  //  * ragged contexts U[1024, 32768] want short ones, the longest requests'
  //    units otherwise finishing alone: B = 1 / 8 ran 17 / 59 us with 1024,
  //    25 / 69 with 2048 (smaller chunks were slower still), B = 32 / 128 191
  //    / 786 us with 1024, 187 / 745 with 2048, 212 / 801 with 4096;
  //  * a single request gains from chunks below 1024 tokens once 1024 leaves
  //    CUs without a unit, up to one unit per CU: 8 KV heads, 2048 / 4096 /
  //    8192 / 16384 / 22656 / 32768 tokens ran 10.7 / 10.1 / 11.4 / 14.1 /
  //    16.1 / 19.1 us with 128 / 128 / 256 / 512 / 768 / 1024-token chunks
  //    against 14.4 / 15.6 / 17.0 / 18.3 / 17.2 / 19.1 with 1024 (four new
  //    tokens, FP8 codes and head_dim 128 alike); more units than CUs cost
  //    more in set-up and merge work than they gain (8192 tokens in 128-token
  //    chunks: 13.5 us).
  (void)head_dim;
  const int64_t simds = (int64_t)cus * 4;
  auto units = [&](int split) { return column_units * ((max_len + split - 1) / split); };
  if (uniform) {
    int split = 8192;
    while (split > 1024 && (split / 2 >= max_len || units(split) < simds / 4)) split /= 2;
    if (split == 1024 && units(1024) < simds / 4 && column_units > 0 && column_units <= cus) {
      // the shortest multiple of 128 tokens that keeps the units within one
      // per CU
      const int64_t per = cus / column_units;     // chunks per (request, KV head, slice)
      const int64_t c = ((max_len + per - 1) / per + 127) / 128 * 128;
      split = (int)(c > 1024 ? 1024 : c);
    }
    return split;
  }
  return units(2048) >= 4 * simds ? 2048 : 1024;
}

template <int D, int CB, bool F8, bool PG>
hipError_t launch_decode_cb(const DecodeArgs& a, int64_t num_units, int waves, hipStream_t stream) {
  const dim3 grid((unsigned)num_units);
  switch (waves) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, CB, 1, F8, PG>), grid, dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, CB, 2, F8, PG>), grid, dim3(128), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_split_kernel<D, CB, 4, F8, PG>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int D, bool F8, bool PG>
hipError_t launch_decode_d(const DecodeArgs& a, int64_t num_units, hipStream_t stream) {
  const int cb = decode_column_blocks(a.ncols, D);
  const int waves = decode_waves_per_unit(num_units, D, cb);
  switch (cb) {
    case 1: return launch_decode_cb<D, 1, F8, PG>(a, num_units, waves, stream);
    case 2: return launch_decode_cb<D, 2, F8, PG>(a, num_units, waves, stream);
    default:
      if constexpr (D == 64) return launch_decode_cb<D, 4, F8, PG>(a, num_units, waves, stream);
      return hipErrorInvalidValue;
  }
}

template <bool F8, bool PG>
hipError_t launch_decode_kind(const DecodeArgs& a, int head_dim, int64_t num_blocks, hipStream_t stream) {
  return head_dim == 64 ? launch_decode_d<64, F8, PG>(a, num_blocks, stream)
                        : launch_decode_d<128, F8, PG>(a, num_blocks, stream);
}

hipError_t launch_decode_split(const DecodeArgs& a, int head_dim, int64_t num_blocks,
                               hipStream_t stream) {
  const bool f8 = a.k_scale != nullptr, pg = a.block_tables != nullptr;
  if (f8) return pg ? launch_decode_kind<true, true>(a, head_dim, num_blocks, stream)
                    : launch_decode_kind<true, false>(a, head_dim, num_blocks, stream);
  return pg ? launch_decode_kind<false, true>(a, head_dim, num_blocks, stream)
            : launch_decode_kind<false, false>(a, head_dim, num_blocks, stream);
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  const dim3 block(kThreads);
  if (a.num_splits <= kMergeBlock && reinterpret_cast<uintptr_t>(a.part_o) % 16 == 0) {
    const int rows_per_block = (kThreads / 64) * (64 / (head_dim / 4));
    const dim3 grid((unsigned)((a.rows + rows_per_block - 1) / rows_per_block));
    if (head_dim == 64)
      hipLaunchKernelGGL(merge_rows_kernel<64>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(merge_rows_kernel<128>, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
