// Multi-row block-sparse attend for gfx950: several token rows that share KV
// pages read and widen each shared page once.
//
// What is computed is exactly the attend of msa_attend.hip (each token row
// attends, per kv head, the causally visible keys of its selected 128-token
// pages; vLLM API page "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparseImpl and the prefill call of MiniMaxM3SparseTritonImpl.forward;
// vLLM test file test_minimax_m3_msa_cutlass_sparse_decode.py, _make_topk),
// plus the dense variant in which every visible block is selected (TensorRT-LLM
// PR #17171, dense-decode commit: the first layers attend the whole page
// table).
//
// Work decomposition.  A workgroup takes a tile of kM token rows for one kv
// head.  As in the single-row attend, wavefront w owns keys [32w, 32w+32) of
// every page and streams them through the same two-deep register ring.  Per
// page it widens its K quarter once (when q is bf16) and runs, for each row
// of the tile that sees the page, S^T = K Q^T, the mask and the lazily
// rescaled online softmax; it then builds its V^T operands once and runs
// O^T += V^T P^T for those rows.  The rows' states from the four
// wavefronts are merged through LDS at the end, row by row.
// The tile's page list is
//  * sparse: the union of the rows' top-k selections, keyed by physical page
//    (rows of different requests may share a tile; a page named by several
//    rows is read once), with each row's visible count;
//  * dense: every block 0..last of one request (tiles never cross requests;
//    tiles after the requests' hold the padding rows), staged into LDS in
//    chunks of kMaxUnion table entries.
// Split-K over the page list writes the same fp32 partials as the single-row
// attend, merged by the same kernel.
#include <climits>

#include "msa_device.h"
#include "msa_internal.h"
#include "msa_page.h"
#include "msa_rows.h"

namespace msa {
namespace {

// The token row of tile position w (-1 when the position holds no row).
__device__ __forceinline__ int tile_row(const AttendParams& p, int tile, int w, int kM) {
  if (p.tile_dense) {
    // Request-aligned tiles: request r owns tiles r*tpr .. r*tpr + tpr - 1;
    // the tiles after the requests' hold the padding rows.
    const int tpr = (p.dql + kM - 1) / kM;
    const int req_tiles = (p.real_rows / p.dql) * tpr;
    if (tile >= req_tiles) {
      const int t = p.real_rows + (tile - req_tiles) * kM + w;
      return t < p.num_rows ? t : -1;
    }
    const int r = tile / tpr;
    const int local = (tile - r * tpr) * kM + w;
    return local < p.dql ? r * p.dql + local : -1;
  }
  return tile * kM + w;
}

// Longest request first.  The workgroups of a launch start in dispatch order
// and a CU holds two at a time, so when requests differ in cost (a ragged
// batch: long requests' tiles see up to twice the pages of short ones) the
// launch ends with the expensive tiles that happened to start last.  Ranking
// the requests by length and giving dispatch position i the tiles of the
// request of rank i puts the long ones first (a list-scheduling model of
// the ragged dql-32 workload: 84 -> 73 us).  Every wavefront ranks the
// requests itself, from one 64-lane load of the lengths and a shuffle loop,
// so no LDS or barrier is needed; ties go to the lower request.  `tile` is
// the dispatch-order tile; returns the tile to process.
template <int kM>
__device__ __forceinline__ int len_ordered_tile(const AttendParams& p, int tile) {
  const int tpr = p.dql / kM;                  // tiles per request (plan: dql % kM == 0)
  const int nreq = p.real_rows / p.dql;        // <= 64 (plan)
  if (tile >= nreq * tpr) return tile;         // padding rows' tiles
  const int want = tile / tpr;
  const int lane = threadIdx.x & 63;
  const int len = lane < nreq ? p.seq_lens[lane] : INT_MIN;
  int rank = 0;
  for (int i = 0; i < nreq; ++i) {
    const int li = __shfl(len, i);
    rank += (li > len) | ((li == len) & (i < lane));
  }
  const uint64_t m = __ballot(lane < nreq && rank == want);
  return (int)__builtin_ctzll(m) * tpr + (tile - want * tpr);
}

// The first half of one page for one row of the tile: S^T from the widened
// K operands (or the K codes, fp8 q), the row's mask and the online softmax
// step; returns the row's P^T operand.  The P V half runs after every row's
// first half, so the widened K and the V^T operands are never live together.
template <int kKv, int kQ>
__device__ __forceinline__ bf16x8_t row_scores(const PageRegs<kv_kind(kKv)>& r,
                                               const bf16x8_t (&kf)[2][4], const QRegs<kQ>& q,
                                               uint32_t ksh, int kbase, int nvis, int g,
                                               float scale_log2, float& m_run, float& l_part,
                                               f32x4_t (&o)[8]) {
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t s[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    if constexpr (kQ == kQE4m3) {
      s[tau] = score_tile_fp8q<kKv>(r, q, tau, ksh);
    } else {
      s[tau] = zero;
#pragma unroll
      for (int c = 0; c < 4; ++c) s[tau] = mfma_bf16_16x16x32(kf[tau][c], q.f[c], s[tau]);
    }
  }
  float z[8];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
    for (int i = 0; i < 4; ++i) z[4 * tau + i] = s[tau][i];
  }
  if (kbase + kKeysPerWave > nvis) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kbase + 16 * tau + 4 * g + i >= nvis) z[4 * tau + i] = -INFINITY;
    }
  }
  return softmax_step(z, scale_log2, m_run, l_part, o);
}

// kOcc3 (2-row tiles over ragged prefill rows): three wavefronts per SIMD,
// with no page prefetch inside a wavefront, so the register file holds a
// third workgroup's wavefronts instead of a second page per wavefront.
// Prefill tiles share few pages (about 1.2 rows per page on the
// chunked-prefill workload), so each workgroup's page loop is bound by its
// own dependent chain and a third workgroup per compute unit pays: 615
// against 640 us there.  Decode tiles (the ragged dql-32 workload) keep two
// wavefronts and the two-deep ring: its long requests' phase needs the
// prefetch (86 against 83 us the other way).  bf16 caches keep it too
// (their wider pages would spill at 168 VGPRs).
template <int kKv, int kQ, int kM, bool kOcc3>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kOcc3 ? 3 : 1, kOcc3 ? 3 : 8)))
void multi_kernel(AttendParams p) {
  constexpr int kKind = kv_kind(kKv);
  constexpr int kRing = kOcc3 ? 1 : kDepth;   // pages per wavefront in the ring
  // Page list entry: (physical page, or 0 when no row sees the entry;
  // byte w = visible rows of the page for tile row w, 0 when it does not see
  // it).  One 8-byte LDS read per page gives its loads and every row's mask.
  __shared__ int2 s_list[kMaxUnion];
  // The rows' selections: entry (row w, slot j) at w * kMaxTopk + j.
  __shared__ __align__(16) int32_t s_ent_page[kMaxUnion];
  __shared__ __align__(16) int32_t s_ent_nv[kMaxUnion];
  __shared__ int32_t s_row_r[kMaxTileRows], s_row_pos[kMaxTileRows];
  __shared__ int32_t s_wave_cnt[kWaves];
  __shared__ int32_t s_nlist;
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][kHeadDim + kOPad];
  // 2-row tiles read q per row and page from LDS ([row][q head][bytes], each
  // head's row padded by 16 bytes so the 16 heads' 16-byte operand reads fall
  // in different banks), so q holds no registers across the page loop: pf1
  // 652 -> 637 us.  4-row tiles keep q in registers (reading it from LDS made
  // d1 6% slower).
  constexpr bool kQInLds = kM == 2;
  constexpr int kQBytes = kHeadDim * (kQ == kQE4m3 ? 1 : 2);
  constexpr int kQStride = kQBytes + 16;
  __shared__ __align__(16) uint8_t s_q[kQInLds ? kM : 1][16][kQStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (tile, kv head, split); all splits of a (tile, head) share
  // an XCD slot.
  const int xslot = blockIdx.x % kXcdSlots;
  const int q8 = blockIdx.x / kXcdSlots;
  const int split = q8 % p.splits;
  const int unit = p.tile_dense ? (q8 / p.splits) * kXcdSlots + xslot
                                : tile_block_unit(p.num_units / p.hkv, p.hkv, xslot,
                                                  q8 / p.splits);
  if (unit < 0 || unit >= p.num_units) return;
  const int h = unit % p.hkv;
  const int tile = p.len_order ? len_ordered_tile<kM>(p, unit / p.hkv) : unit / p.hkv;
  const int head0 = h * p.group;

  // Prologue.  Everything the page list needs is requested before anything
  // waits: each (row, slot) thread's top-k entry and its row's length, and
  // the q staging loads (q of every row in range is staged; rows found dead
  // below never read it).  Then the block-table entries of the visible
  // slots; then the list is built in LDS.  Two dependent memory round trips
  // before the first page's loads, where looking the rows up first, then
  // staging q, then reading the top-k entries took four.
  const int k = p.topk_k;
  const int ew = tid / kMaxTopk;           // this thread's (row, slot) entry
  const int ej = tid - ew * kMaxTopk;
  const bool has_entry = !p.tile_dense && ew < kM;
  const int et = has_entry ? tile_row(p, tile, ew, kM) : -1;
  int b_raw = -1;
  if (has_entry && ej < k && et >= 0 && et < p.num_rows)
    b_raw = p.topk[et * p.tk_s0 + h * p.tk_s1 + ej * p.tk_s2];
  constexpr int kQChunks = kQBytes / 16;
  constexpr int kQLoads = (kM * 16 * kQChunks + kThreads - 1) / kThreads;
  u32x4_t qv[kQInLds ? kQLoads : 1];
#pragma unroll
  for (int i = 0; i < (kQInLds ? kQLoads : 0); ++i) {
    const int c = tid + i * kThreads;
    const int w = c / (16 * kQChunks);
    const int rem = c - w * (16 * kQChunks);
    const int qh = rem / kQChunks;
    const int off = (rem - qh * kQChunks) * 16;
    const int t = w < kM ? tile_row(p, tile, w, kM) : -1;
    qv[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (t >= 0 && t < p.num_rows && qh < p.group)
      qv[i] = *reinterpret_cast<const u32x4_t*>(p.q + ((int64_t)t * p.hq + head0 + qh) *
                                                          kQBytes + off);
  }
  // The row of this thread's entry (sparse), or of thread w < kM (dense).
  const int lw = p.tile_dense ? tid : ew;
  const int lt = p.tile_dense ? (tid < kM ? tile_row(p, tile, tid, kM) : -1) : et;
  int row_r = -1, row_pos = -1;
  if (lt >= 0 && lt < p.num_rows && lw < kM) {
    int rr = 0, pp = 0;
    if (locate_token(p, lt, rr, pp)) {
      row_r = rr;
      row_pos = pp;
    }
  }
  if (lw < kM && (p.tile_dense || ej == 0)) {
    s_row_r[lw] = row_r;
    s_row_pos[lw] = row_pos;
  }
#pragma unroll
  for (int i = 0; i < (kQInLds ? kQLoads : 0); ++i) {
    const int c = tid + i * kThreads;
    if (c < kM * 16 * kQChunks) {
      const int w = c / (16 * kQChunks);
      const int rem = c - w * (16 * kQChunks);
      const int qh = rem / kQChunks;
      const int off = (rem - qh * kQChunks) * 16;
      *reinterpret_cast<u32x4_t*>(&s_q[kQInLds ? w : 0][qh][off]) = qv[i];
    }
  }

  int npages;
  int dense_r = -1, dense_pos_max = -1;
  if (!p.tile_dense) {
    // Union of the rows' selections: thread (row w, slot j) stages its entry
    // (page -1 for an empty, invalid or padding slot) at w * kMaxTopk + j.
    const int kq = (k + 3) & ~3;  // slots scanned per row (the pad is -1)
    int page = -1, nv = 0;
    if (has_entry) {
      const int b = b_raw;
      if (row_r >= 0 && (b >= 0) & (b < p.bt_stride) & ((int64_t)b * kPage <= row_pos)) {
        const int pg = p.block_table[(int64_t)row_r * p.bt_stride + b];
        if (pg >= 0 && pg < p.num_kv_blocks) {
          page = pg;
          nv = min(kPage, row_pos - b * kPage + 1);
        }
      }
      s_ent_page[tid] = page;
      s_ent_nv[tid] = nv;
    }
    __syncthreads();
    // One pass over every staged entry, four at a time: the first entry (in
    // (row, slot) order) naming this entry's page, and each row's largest
    // visible count for that page.  The first occurrence opens a list slot.
    bool first = false;
    uint32_t nv4 = 0;
    if (page >= 0) {
      int first_e = tid;
#pragma unroll
      for (int w = 0; w < kM; ++w) {
        int v = 0;
        for (int j = 0; j < kq; j += 4) {
          const int e2 = w * kMaxTopk + j;
          const int4 pg4 = *reinterpret_cast<const int4*>(&s_ent_page[e2]);
          const int4 nv4v = *reinterpret_cast<const int4*>(&s_ent_nv[e2]);
          if (pg4.x == page) { first_e = min(first_e, e2); v = max(v, nv4v.x); }
          if (pg4.y == page) { first_e = min(first_e, e2 + 1); v = max(v, nv4v.y); }
          if (pg4.z == page) { first_e = min(first_e, e2 + 2); v = max(v, nv4v.z); }
          if (pg4.w == page) { first_e = min(first_e, e2 + 3); v = max(v, nv4v.w); }
        }
        nv4 |= (uint32_t)v << (8 * w);
      }
      first = first_e == tid;
    }
    // Slots follow entry order (a prefix count over the waves).  (Ordering
    // them by logical block, so that a request's tiles meet on shared pages
    // in L2, cut reads beyond L2 on the ragged dql-32 workload from 1.59x to
    // 1.00x of its unique bytes but made the step slower: tiles walking the
    // same pages in step miss together.)
    const uint64_t bal = __ballot(first);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += s_wave_cnt[w2];
    if (first) {
      const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
      s_list[slot] = make_int2(page, (int)nv4);
    }
    if (tid == 0) {
      int tot = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) tot += s_wave_cnt[w2];
      s_nlist = tot;
    }
    __syncthreads();
    npages = s_nlist;
  } else {
    __syncthreads();  // the rows' lookups are in s_row_r / s_row_pos
    dense_r = s_row_r[0];
#pragma unroll
    for (int w = 0; w < kM; ++w) dense_pos_max = max(dense_pos_max, s_row_pos[w]);
    npages = dense_r >= 0 && dense_pos_max >= 0
                 ? min(dense_pos_max / kPage + 1, p.bt_stride)
                 : 0;
  }

  // This split's share of the page list.
  const int lo = (int)((int64_t)npages * split / p.splits);
  const int hi = (int)((int64_t)npages * (split + 1) / p.splits);

  // Q^T of every row of the tile (zeros for dead rows and q rows >= G).

  // 4-row tiles: Q^T of every row in registers (zeros for dead rows and q
  // rows >= G).
  QRegs<kQ> qf[kQInLds ? 1 : kM];
  if constexpr (!kQInLds) {
#pragma unroll
    for (int w = 0; w < kM; ++w) {
      const bool load = s_row_r[w] >= 0 && n < p.group;
      const int64_t q_row = (int64_t)(load ? tile_row(p, tile, w, kM) : 0) * p.hq + head0 + n;
      load_q_operand<kKind, kQ>(qf[w], p.q + q_row * kQBytes, load, g);
    }
  }

  float m_run[kM], l_part[kM];
  f32x4_t o[kM][8];
#pragma unroll
  for (int w = 0; w < kM; ++w) {
    m_run[w] = -INFINITY;
    l_part[w] = 0.f;
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) o[w][t8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int kbase = wave * kKeysPerWave;
  const uint8_t* head_base = p.kv + h * p.kv_s1;
  const uint32_t row_stride = (uint32_t)p.kv_s2;
  // 2-row decode tiles read each page through a buffer descriptor bounded at
  // the tile's largest visible count (zeros past it, the lane offsets fixed
  // for the launch), as the single-row attend does: c4 82.7 -> 81.5 us.  The
  // other tiles keep the clamped loads: the launch-long lane offsets add
  // spills to the three-wave prefill tiles (pf1 613 -> 621 us), and the 4-row
  // dense tiles ran 316 -> 368 us with them.
  constexpr bool kBoundedLoads = kM == 2 && !kOcc3;
  // 2-row tiles read 8-bit K whole-row and move it into the MFMA's layout
  // through the wavefront's part of the merge buffer, which the page loop
  // does not otherwise use (k8_whole_to_mfma): chunked prefill 617 -> 557 us,
  // ragged dql-32 decode 81.9 -> 80.8 us.  The 4-row dense tiles, one
  // wavefront per SIMD, lose more to the LDS round trip in their page chain
  // than they gain (322 -> 336 us), and keep the MFMA-layout loads.
  constexpr bool kWholeK = kKind == 1 && kM == 2;
  uint8_t* k_scratch = reinterpret_cast<uint8_t*>(&s_o[wave][0][0]);
  LaneRows lr = lane_rows<kKind, kWholeK>(kbase, n, g);
  if constexpr (kBoundedLoads) lane_offsets(lr, row_stride);
  const int32_t* dense_row =
      p.block_table + (int64_t)(dense_r >= 0 ? dense_r : 0) * p.bt_stride;

  // The page list in chunks of kMaxUnion entries (a sparse list is a single,
  // already staged chunk; dense chunks are staged here from the table).
  for (int c0 = lo; c0 < hi; c0 += kMaxUnion) {
    const int c1 = min(hi, c0 + kMaxUnion);
    if (p.tile_dense) {
      __syncthreads();  // the previous chunk's entries are no longer read
      for (int u = c0 + tid; u < c1; u += kThreads) {
        const int raw = dense_row[u];
        const bool ok = raw >= 0 && raw < p.num_kv_blocks;
        uint32_t nv4 = 0;
#pragma unroll
        for (int w = 0; w < kM; ++w) {
          int v = 0;
          if (ok && s_row_pos[w] >= 0) v = max(0, min(kPage, s_row_pos[w] - u * kPage + 1));
          nv4 |= (uint32_t)v << (8 * w);
        }
        s_list[u - c0] = make_int2(nv4 != 0 ? raw : 0, (int)nv4);
      }
      __syncthreads();
    }
    const int base = p.tile_dense ? c0 : 0;  // list index of LDS entry 0
    // Issues the loads of list entry u into `r` and returns the entry's row
    // bytes (wave-uniform), kept in scalar registers until the page is used.
    auto fetch = [&](int u, PageRegs<kKind>& r) -> uint32_t {
      const int2 e = s_list[u - base];
      const int pg = __builtin_amdgcn_readfirstlane(e.x);
      const uint32_t nv4 = (uint32_t)__builtin_amdgcn_readfirstlane(e.y);
      uint32_t vmax = 0;
#pragma unroll
      for (int w = 0; w < kM; ++w) vmax = max(vmax, (nv4 >> (8 * w)) & 0xffu);
      if constexpr (kBoundedLoads)
        load_page_rows<kKind, kWholeK>(r, head_base + (int64_t)pg * p.kv_s0, row_stride,
                                       (int)vmax, lr);
      else
        load_page<kKind, kWholeK>(r, head_base + (int64_t)pg * p.kv_s0, row_stride,
                                  (int)max(vmax, 1u) - 1, lr);
      return nv4;
    };

    PageRegs<kKind> buf[kRing];
    uint32_t bnv[kRing];
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j) bnv[j] = fetch(min(c0 + j, c1 - 1), buf[j]);
    for (int i = c0;; i += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) {
        const int cur = i + j;
        if (cur >= c1) goto chunk_done;
        {
          const int nx = (j + kRing - 1) % kRing;
          bnv[nx] = fetch(min(cur + kRing - 1, c1 - 1), buf[nx]);
          const uint32_t nv4 = bnv[j];
          bool any = false;
#pragma unroll
          for (int w = 0; w < kM; ++w) any |= (int)((nv4 >> (8 * w)) & 0xffu) > kbase;
          if (any) {
            if constexpr (kWholeK) k8_whole_to_mfma(buf[j], k_scratch, n, g);
            // This wavefront's keys are widened once for all rows of the
            // tile: K first, for every row's S^T and softmax; then V, for
            // every row's P V.
            bf16x8_t pb[kM];
            {
              bf16x8_t kf[2][4];
              if constexpr (kQ != kQE4m3) {
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
                  widen_k_tile<kKv>(buf[j], tau, lr.ksh, kf[tau]);
              }
#pragma unroll
              for (int w = 0; w < kM; ++w) {
                const int nv = (int)((nv4 >> (8 * w)) & 0xffu);
                if (nv > kbase) {
                  if constexpr (kQInLds) {
                    QRegs<kQ> qw;
                    load_q_operand<kKind, kQ>(qw, &s_q[w][n][0], true, g);
                    pb[w] = row_scores<kKv, kQ>(buf[j], kf, qw, lr.ksh, kbase, nv, g,
                                                p.scale_log2, m_run[w], l_part[w], o[w]);
                  } else {
                    pb[w] = row_scores<kKv, kQ>(buf[j], kf, qf[w], lr.ksh, kbase, nv, g,
                                                p.scale_log2, m_run[w], l_part[w], o[w]);
                  }
                }
              }
            }
            u32x4_t vt[8];
            build_vt<kKv>(buf[j], lr.vsh, vt);
#pragma unroll
            for (int w = 0; w < kM; ++w) {
              if ((int)((nv4 >> (8 * w)) & 0xffu) > kbase) {
#pragma unroll
                for (int t8 = 0; t8 < 8; ++t8)
                  o[w][t8] = mfma_bf16_16x16x32(as_bf16x8(vt[t8]), pb[w], o[w][t8]);
              }
            }
          }
        }
      }
    }
  chunk_done:;
  }

  // Row by row: merge the four wavefronts' states, then write the bf16 row
  // (one split), the fp32 partial (several), or zeros for a padding row.
  const int qr = tid >> 4;
  const int d0 = (tid & 15) * 8;
#pragma unroll
  for (int w = 0; w < kM; ++w) {
    const int t = tile_row(p, tile, w, kM);
    const bool live = s_row_r[w] >= 0;
    const float l_run = wave_sum_xor_16_32(l_part[w]);
    __syncthreads();  // the previous row's merge buffers are no longer read
    if (g == 0) {
      s_m[wave][n] = m_run[w];
      s_l[wave][n] = l_run;
    }
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + t8] = o[w][t8][i];
    }
    __syncthreads();
    if (t < 0 || t >= p.num_rows || qr >= p.group) continue;
    const int64_t row = (int64_t)t * p.hq + head0 + qr;
    if (!live) {
      if (split == 0) {
        *reinterpret_cast<u32x4_t*>(p.out + row * kHeadDim + d0) = u32x4_t{0u, 0u, 0u, 0u};
      }
      continue;
    }
    float mw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      mw[w2] = s_m[w2][qr];
      M = fmaxf(M, mw[w2]);
    }
    float L = 0.f;
    float acc[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) acc[kk] = 0.f;
    // An empty wavefront weighs 0 (multiplied in, so a NaN sum propagates).
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const float e = mw[w2] == -INFINITY ? 0.f : fast_exp2(mw[w2] - M);
      L += e * s_l[w2][qr];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) acc[kk] += e * s_o[w2][qr][d0 + kk];
    }
    if (p.splits == 1) {
      store_row(p.out + row * kHeadDim + d0, acc, L, p.v_scale);
    } else {
      float* po = p.part_o + (row * p.splits + split) * kHeadDim + d0;
      *reinterpret_cast<f32x4_t*>(po) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4_t*>(po + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
      if (d0 == 0) {
        float* pml = p.part_ml + (row * p.splits + split) * 2;
        pml[0] = M;
        pml[1] = L;
      }
    }
  }
}

template <int kKv, int kQ>
hipError_t launch_tile_fmt(const AttendParams& p, int tile_rows, dim3 gd, hipStream_t stream) {
  if (tile_rows == 4)
    hipLaunchKernelGGL((multi_kernel<kKv, kQ, 4, false>), gd, dim3(kThreads), 0, stream, p);
  else if (kKv != kKvBf16 && p.cu_q != nullptr)  // bf16 pages would spill at 168 VGPRs
    hipLaunchKernelGGL((multi_kernel<kKv, kQ, 2, kKv != kKvBf16>), gd, dim3(kThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((multi_kernel<kKv, kQ, 2, false>), gd, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile(const AttendParams& p, int kv_fmt, int q_fmt, int tile_rows,
                       hipStream_t stream) {
  // Dense tiles keep the plain round robin (a dense tile's rows share every
  // page of one request; tiles of different requests share none).
  const int64_t groups = p.tile_dense ? ((int64_t)p.num_units + kXcdSlots - 1) / kXcdSlots
                                      : tile_block_groups(p.num_units / p.hkv, p.hkv);
  const int64_t grid = groups * kXcdSlots * p.splits;
  if (grid <= 0) return hipSuccess;
  const dim3 gd((uint32_t)grid);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3) return launch_tile_fmt<kKvE4m3, kQE4m3>(p, tile_rows, gd, stream);
    if (kv_fmt == kKvE5m2) return launch_tile_fmt<kKvE5m2, kQE4m3>(p, tile_rows, gd, stream);
    if (kv_fmt == kKvMxfp4) return launch_tile_fmt<kKvMxfp4, kQE4m3>(p, tile_rows, gd, stream);
    return hipErrorInvalidValue;
  }
  if (kv_fmt == kKvE4m3) return launch_tile_fmt<kKvE4m3, kQBf16>(p, tile_rows, gd, stream);
  if (kv_fmt == kKvE5m2) return launch_tile_fmt<kKvE5m2, kQBf16>(p, tile_rows, gd, stream);
  if (kv_fmt == kKvMxfp4) return launch_tile_fmt<kKvMxfp4, kQBf16>(p, tile_rows, gd, stream);
  return launch_tile_fmt<kKvBf16, kQBf16>(p, tile_rows, gd, stream);
}

}  // namespace msa
