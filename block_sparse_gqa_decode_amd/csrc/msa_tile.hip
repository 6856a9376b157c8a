// Multi-token block-sparse attend for gfx950: several token rows that share
// KV pages read each shared page once.
//
// What is computed is exactly the attend of msa_attend.hip (each token row
// attends, per kv head, the causally visible keys of its selected 128-token
// pages; vLLM API page "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparseImpl and the prefill call of MiniMaxM3SparseTritonImpl.forward;
// vLLM test file test_minimax_m3_msa_cutlass_sparse_decode.py, _make_topk),
// plus the dense variant in which every visible block is selected (TensorRT-LLM
// PR #17171, dense-decode commit: the first layers attend every block).
//
// Work decomposition.  A workgroup has kW wavefronts and takes a tile of up
// to kW token rows for one kv head; wavefront w owns token row w of the tile
// (its G <= 16 q heads are the 16 columns of the MFMA tiles) and keeps that
// row's whole online-softmax state, so no state is merged across wavefronts.
// The tile's pages are
//  * sparse: the union of the rows' top-k selections, keyed by physical page
//    (rows of different requests may share the tile; a page named by several
//    rows is read once), with per-row visibility;
//  * dense: every block 0..last of one request (tiles never cross requests).
// All threads of the workgroup copy each page (rows up to the largest visible
// count, clamped, so no stale row is read) into a two-slot LDS ring; the
// copy of page i+1 is in flight while the wavefronts compute page i out of
// LDS.  Rows are stored with a 16-byte pad so the 16 key rows of an MFMA tile
// fall in distinct LDS banks.
//
// Per page and wavefront: S^T = K Q^T over 8 tiles of 16 keys (the attend's
// operand layout, K now read from LDS; one 16x16x128 fp8 MFMA per tile with an
// fp8 q), the row's mask (selected by this row and key < its visible count),
// the lazily rescaled online softmax of the attend, then O^T += V^T P^T over 4
// chunks of 32 keys.  Split-K over the tile's page list writes the same fp32
// partials as the attend, merged by the same kernel.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_rows.h"

namespace msa {
namespace {

constexpr float kTileRescaleSlack = 8.0f;

template <bool kFp8>
struct TileGeom {
  static constexpr int kRowBytes = kFp8 ? 256 : 512;   // a packed K|V row
  static constexpr int kPitch = kRowBytes + 16;         // LDS row pitch
  static constexpr int kPageLds = kPage * kPitch;       // one page slot
  static constexpr int kChunks = kPage * kRowBytes / 16;  // 16-byte copies per page
};

__device__ __forceinline__ int tile_key_of_slot(int g, int j) {
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// S^T tile kt (keys 16kt..16kt+15) of the page in LDS for this lane's q row.
template <int kKv, int kQ>
__device__ __forceinline__ f32x4_t lds_score_tile(const uint8_t* pg, int kt, int n, int g,
                                                  const QRegs<kQ>& q) {
  constexpr bool kFp8 = kKv != kKvBf16;
  const uint8_t* row = pg + (kt * 16 + n) * TileGeom<kFp8>::kPitch;
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kFp8) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(row + 16 * g);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(row + 64 + 16 * g);
    if constexpr (kQ == kQE4m3) {
      return mfma_f8_16x16x128<kKv == kKvE5m2 ? 1 : 0, 0>(cat_i32x8(a, b), q.b, zero);
    } else {
      f32x4_t s = zero;
      s = mfma_bf16_16x16x32(as_bf16x8(f8x8_to_bf16x8<kKv>(a.x, a.y)), q.f[0], s);
      s = mfma_bf16_16x16x32(as_bf16x8(f8x8_to_bf16x8<kKv>(a.z, a.w)), q.f[1], s);
      s = mfma_bf16_16x16x32(as_bf16x8(f8x8_to_bf16x8<kKv>(b.x, b.y)), q.f[2], s);
      s = mfma_bf16_16x16x32(as_bf16x8(f8x8_to_bf16x8<kKv>(b.z, b.w)), q.f[3], s);
      return s;
    }
  } else {
    f32x4_t s = zero;
    s = mfma_bf16_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(row + 32 * g)),
                           q.f[0], s);
    s = mfma_bf16_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(row + 32 * g + 16)),
                           q.f[1], s);
    s = mfma_bf16_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4_t*>(row + 128 + 32 * g)),
                           q.f[2], s);
    s = mfma_bf16_16x16x32(
        as_bf16x8(*reinterpret_cast<const u32x4_t*>(row + 128 + 32 * g + 16)), q.f[3], s);
    return s;
  }
}

// One page of one token row: scores, mask, online softmax, P V.
template <int kKv, int kQ>
__device__ __forceinline__ void tile_page(const uint8_t* pg, const QRegs<kQ>& q, int nvis,
                                          int n, int g, float scale_log2, float& m_run,
                                          float& l_part, f32x4_t (&o)[8]) {
  constexpr bool kFp8 = kKv != kKvBf16;
  float z[32];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const f32x4_t s = lds_score_tile<kKv, kQ>(pg, kt, n, g, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) z[4 * kt + i] = s[i];
  }
  if (nvis < kPage) {
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * kt + 4 * g + i >= nvis) z[4 * kt + i] = -INFINITY;
    }
  }
  float mx = z[0];
#pragma unroll
  for (int e = 1; e < 32; ++e) mx = fmaxf(mx, z[e]);
  mx *= scale_log2;
  // Lazy rescale, as in the single-token attend: the reference point of a row
  // moves only when a score exceeds it by more than the slack.
  if (__any(mx > m_run + kTileRescaleSlack)) {
    const float mrow = wave_max_xor_16_32(mx);
    const float m_new = mrow > m_run + kTileRescaleSlack ? mrow : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    l_part *= alpha;
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) o[t8] *= alpha;
    m_run = m_new;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // P^T of keys 32c..32c+31 from the accumulators of tiles 2c and 2c+1.
    float pz[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pz[e] = fast_exp2(fmaf(z[8 * c + e], scale_log2, -m_run));
    l_part += ((pz[0] + pz[1]) + (pz[2] + pz[3])) + ((pz[4] + pz[5]) + (pz[6] + pz[7]));
    u32x4_t pw;
    pw.x = pack_bf16x2(pz[0], pz[1]);
    pw.y = pack_bf16x2(pz[2], pz[3]);
    pw.z = pack_bf16x2(pz[4], pz[5]);
    pw.w = pack_bf16x2(pz[6], pz[7]);
    const bf16x8_t pb = as_bf16x8(pw);
    // V^T: lane (n, g) takes head dims 8n..8n+7 of its 8 key slots.
    u32x4_t vd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint8_t* row = pg + (32 * c + tile_key_of_slot(g, j)) * TileGeom<kFp8>::kPitch;
      if constexpr (kFp8) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(row + kHeadDim + 8 * n);
        vd[j] = f8x8_to_bf16x8<kKv>(v.x, v.y);
      } else {
        vd[j] = *reinterpret_cast<const u32x4_t*>(row + 2 * kHeadDim + 16 * n);
      }
    }
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      const uint32_t sel = (t8 & 1) ? 0x07060302u : 0x05040100u;
      const int w = t8 >> 1;
      u32x4_t a;
      a.x = byte_perm(vd[1][w], vd[0][w], sel);
      a.y = byte_perm(vd[3][w], vd[2][w], sel);
      a.z = byte_perm(vd[5][w], vd[4][w], sel);
      a.w = byte_perm(vd[7][w], vd[6][w], sel);
      o[t8] = mfma_bf16_16x16x32(as_bf16x8(a), pb, o[t8]);
    }
  }
}

// The token row of tile position w (-1 when the position holds no row).
__device__ __forceinline__ int tile_row(const AttendParams& p, int tile, int w, int kW) {
  if (p.tile_dense) {
    // Request-aligned tiles: request r owns tiles r*tpr .. r*tpr + tpr - 1;
    // the tiles after the requests' hold the padding rows.
    const int tpr = (p.dql + kW - 1) / kW;
    const int req_tiles = (p.real_rows / p.dql) * tpr;
    if (tile >= req_tiles) {
      const int t = p.real_rows + (tile - req_tiles) * kW + w;
      return t < p.num_rows ? t : -1;
    }
    const int r = tile / tpr;
    const int local = (tile - r * tpr) * kW + w;
    return local < p.dql ? r * p.dql + local : -1;
  }
  return tile * kW + w;
}

template <int kKv, int kQ, int kW>
__global__ __launch_bounds__(64 * kW) void tile_kernel(AttendParams p) {
  constexpr bool kFp8 = kKv != kKvBf16;
  using Geom = TileGeom<kFp8>;
  constexpr int kThreadsT = 64 * kW;
  constexpr int kPerThread = Geom::kChunks / kThreadsT;
  static_assert(Geom::kChunks % kThreadsT == 0, "page copy must divide evenly");

  __shared__ __align__(16) uint8_t s_buf[2 * Geom::kPageLds];   // 2 page slots
  __shared__ int32_t s_upage[kMaxUnion];                // union: physical page
  __shared__ uint8_t s_unv[kMaxUnion][kMaxTileRows];    // union: visible rows per row
  __shared__ int32_t s_ent_page[kMaxUnion];
  __shared__ int32_t s_ent_nv[kMaxUnion];
  __shared__ int32_t s_row_r[kMaxTileRows], s_row_pos[kMaxTileRows];
  __shared__ int32_t s_wave_cnt[kMaxTileRows];
  __shared__ int32_t s_nunion;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (tile, kv head, split), all splits of a (tile, head) on one
  // XCD slot.
  const int xslot = blockIdx.x % kXcdSlots;
  const int q8 = blockIdx.x / kXcdSlots;
  const int split = q8 % p.splits;
  const int unit = (q8 / p.splits) * kXcdSlots + xslot;
  if (unit >= p.num_units) return;
  const int tile = unit / p.hkv;
  const int h = unit - tile * p.hkv;
  const int head0 = h * p.group;

  // Rows of the tile.
  if (tid < kW) {
    const int t = tile_row(p, tile, tid, kW);
    int r = -1, pos = -1;
    if (t >= 0 && t < p.num_rows) {
      int rr = 0, pp = 0;
      if (locate_token(p, t, rr, pp)) {
        r = rr;
        pos = pp;
      }
    }
    s_row_r[tid] = r;
    s_row_pos[tid] = pos;
  }
  __syncthreads();

  // The tile's page list: sparse = union of the rows' selections; dense =
  // blocks 0..last of the tile's request.
  int npages;
  int dense_r = -1, dense_pos_max = -1;
  if (!p.tile_dense) {
    const int k = p.topk_k;
    const int e = tid;
    int page = -1, nv = 0;
    if (e < kW * k) {
      const int w = e / k;
      const int j = e - w * k;
      const int r = s_row_r[w];
      const int pos = s_row_pos[w];
      const int t = tile_row(p, tile, w, kW);
      if (r >= 0) {
        const int b = p.topk[t * p.tk_s0 + h * p.tk_s1 + j * p.tk_s2];
        if (b >= 0 && b < p.bt_stride && (int64_t)b * kPage <= pos) {
          const int pg = p.block_table[(int64_t)r * p.bt_stride + b];
          if (pg >= 0 && pg < p.num_kv_blocks) {
            page = pg;
            nv = min(kPage, pos - b * kPage + 1);
          }
        }
      }
      s_ent_page[e] = page;
      s_ent_nv[e] = nv;
    }
    __syncthreads();
    // First occurrence of each page opens a union slot; slots follow entry
    // order (a prefix count over the workgroup's waves).
    bool first = false;
    if (e < kW * k && page >= 0) {
      first = true;
      for (int e2 = 0; e2 < e; ++e2)
        if (s_ent_page[e2] == page) {
          first = false;
          break;
        }
    }
    const uint64_t bal = __ballot(first);
    if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += s_wave_cnt[w2];
    if (first) {
      const int slot = base + __popcll(bal & ((1ull << lane) - 1ull));
      s_upage[slot] = page;
      for (int w = 0; w < kW; ++w) {
        int v = 0;
        for (int j = 0; j < k; ++j) {
          const int e2 = w * k + j;
          if (s_ent_page[e2] == page) v = max(v, s_ent_nv[e2]);
        }
        s_unv[slot][w] = (uint8_t)v;
      }
    }
    if (tid == 0) {
      int tot = 0;
      for (int w2 = 0; w2 < kW; ++w2) tot += s_wave_cnt[w2];
      s_nunion = tot;
    }
    __syncthreads();
    npages = s_nunion;
  } else {
    dense_r = s_row_r[0];
    for (int w = 0; w < kW; ++w) dense_pos_max = max(dense_pos_max, s_row_pos[w]);
    npages = dense_r >= 0 && dense_pos_max >= 0
                 ? min(dense_pos_max / kPage + 1, p.bt_stride)
                 : 0;
  }

  // This split's share of the page list.
  const int lo = (int)((int64_t)npages * split / p.splits);
  const int hi = (int)((int64_t)npages * (split + 1) / p.splits);

  // Page u of the list: physical page (or -1) and this row's / the largest
  // visible row count.  Dense pages come from the table entry `raw`, read two
  // pages ahead so the copy of a page never waits on its own table read.
  const int my_pos = s_row_pos[wave];
  const int32_t* dense_row =
      p.block_table + (int64_t)(dense_r >= 0 ? dense_r : 0) * p.bt_stride;
  auto page_info = [&](int u, int raw, int& pg, int& nv_me, int& nv_max) {
    if (!p.tile_dense) {
      pg = s_upage[u];
      nv_me = s_unv[u][wave];
      nv_max = 0;
#pragma unroll
      for (int w = 0; w < kW; ++w) nv_max = max(nv_max, (int)s_unv[u][w]);
    } else {
      pg = raw >= 0 && raw < p.num_kv_blocks ? raw : -1;
      nv_me = my_pos >= 0 ? max(0, min(kPage, my_pos - u * kPage + 1)) : 0;
      nv_max = max(0, min(kPage, dense_pos_max - u * kPage + 1));
      if (pg < 0) nv_me = nv_max = 0;
    }
  };

  // Q^T of this wavefront's row.
  const int my_row = tile_row(p, tile, wave, kW);
  const bool row_live = s_row_r[wave] >= 0;
  QRegs<kQ> qf;
  {
    const int64_t q_row = (int64_t)(row_live ? my_row : 0) * p.hq + head0 + n;
    const bool load = row_live && n < p.group;
    if constexpr (kQ == kQE4m3) {
      u32x4_t a = u32x4_t{0u, 0u, 0u, 0u}, b = a;
      if (load) {
        const uint8_t* qp = p.q + q_row * kHeadDim;
        a = *reinterpret_cast<const u32x4_t*>(qp + 16 * g);
        b = *reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g);
      }
      qf.b = cat_i32x8(a, b);
    } else {
      if (load) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + q_row * kHeadDim;
        qf.f[0] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 16 * g));
        qf.f[1] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 16 * g + 8));
        qf.f[2] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g));
        qf.f[3] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g + 8));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) qf.f[c] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
      }
    }
  }

  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) o[t8] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint8_t* head_base = p.kv + h * p.kv_s1;
  const uint32_t row_stride = (uint32_t)p.kv_s2;

  // Copy registers of one page: chunk c = tid + kThreadsT*i is row c / (row
  // bytes / 16), 16-byte column c % (row bytes / 16); rows at or past the
  // largest visible count repeat the last visible row.
  u32x4_t cp[kPerThread];
  auto issue_copy = [&](int u, int raw) {
    int pg, nv_me, nv_max;
    page_info(u, raw, pg, nv_me, nv_max);
    const int lim = max(nv_max, 1) - 1;
    const uint8_t* src = head_base + (int64_t)(pg >= 0 ? pg : 0) * p.kv_s0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + kThreadsT * i;
      const int row = c / (Geom::kRowBytes / 16);
      const int col = c - row * (Geom::kRowBytes / 16);
      cp[i] = *reinterpret_cast<const u32x4_t*>(src + (uint32_t)min(row, lim) * row_stride +
                                                16u * col);
    }
  };
  auto store_copy = [&](int slot) {
    uint8_t* dst = s_buf + slot * Geom::kPageLds;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + kThreadsT * i;
      const int row = c / (Geom::kRowBytes / 16);
      const int col = c - row * (Geom::kRowBytes / 16);
      *reinterpret_cast<u32x4_t*>(dst + row * Geom::kPitch + 16 * col) = cp[i];
    }
  };

  // Table entries of pages u and u+1 (dense mode; indexes clamped to the
  // range, so the reads are unconditional and in bounds).
  int tbl_cur = 0, tbl_next = 0;
  if (p.tile_dense && lo < hi) {
    tbl_cur = dense_row[lo];
    tbl_next = dense_row[min(lo + 1, hi - 1)];
  }
  if (lo < hi) issue_copy(lo, tbl_cur);
  for (int u = lo; u < hi; ++u) {
    const int slot = (u - lo) & 1;
    store_copy(slot);
    __syncthreads();
    const int tbl_after = p.tile_dense ? dense_row[min(u + 2, hi - 1)] : 0;
    if (u + 1 < hi) issue_copy(u + 1, tbl_next);
    int pg, nv_me, nv_max;
    page_info(u, tbl_cur, pg, nv_me, nv_max);
    tbl_cur = tbl_next;
    tbl_next = tbl_after;
    if (row_live && nv_me > 0)
      tile_page<kKv, kQ>(s_buf + slot * Geom::kPageLds, qf, nv_me, n, g, p.scale_log2, m_run,
                         l_part, o);
  }

  // Row results: exact zeros for a row with no key; fp32 partials with splits.
  if (!row_live) {
    // A padding row (or a tile position past its request's rows): zeros once.
    if (my_row >= 0 && my_row < p.num_rows && split == 0 && n < p.group) {
      uint16_t* dst = p.out + ((int64_t)my_row * p.hq + head0 + n) * kHeadDim + 32 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4_t*>(dst + 8 * i) = u32x4_t{0u, 0u, 0u, 0u};
    }
    return;
  }
  const float l_run = wave_sum_xor_16_32(l_part);
  if (n >= p.group) return;
  const int64_t row = (int64_t)my_row * p.hq + head0 + n;
  if (p.splits == 1) {
    u32x4_t ov[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (l_run > 0.f) {
      const float inv = p.v_scale / l_run;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ov[i].x = pack_bf16x2(o[0][i] * inv, o[1][i] * inv);
        ov[i].y = pack_bf16x2(o[2][i] * inv, o[3][i] * inv);
        ov[i].z = pack_bf16x2(o[4][i] * inv, o[5][i] * inv);
        ov[i].w = pack_bf16x2(o[6][i] * inv, o[7][i] * inv);
      }
    }
    uint16_t* dst = p.out + row * kHeadDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(dst + 8 * i) = ov[i];
    return;
  }
  float* po = p.part_o + (row * p.splits + split) * kHeadDim + 32 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<f32x4_t*>(po + 8 * i) = f32x4_t{o[0][i], o[1][i], o[2][i], o[3][i]};
    *reinterpret_cast<f32x4_t*>(po + 8 * i + 4) = f32x4_t{o[4][i], o[5][i], o[6][i], o[7][i]};
  }
  if (g == 0) {
    float* pml = p.part_ml + (row * p.splits + split) * 2;
    pml[0] = m_run;
    pml[1] = l_run;
  }
}

template <int kKv, int kQ>
hipError_t launch_tile_fmt(const AttendParams& p, int tile_rows, dim3 gd, hipStream_t stream) {
  if (tile_rows == 8)
    hipLaunchKernelGGL((tile_kernel<kKv, kQ, 8>), gd, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((tile_kernel<kKv, kQ, 4>), gd, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile(const AttendParams& p, int kv_fmt, int q_fmt, int tile_rows,
                       hipStream_t stream) {
  const int64_t groups = ((int64_t)p.num_units + kXcdSlots - 1) / kXcdSlots;
  const int64_t grid = groups * kXcdSlots * p.splits;
  if (grid <= 0) return hipSuccess;
  const dim3 gd((uint32_t)grid);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3) return launch_tile_fmt<kKvE4m3, kQE4m3>(p, tile_rows, gd, stream);
    if (kv_fmt == kKvE5m2) return launch_tile_fmt<kKvE5m2, kQE4m3>(p, tile_rows, gd, stream);
    return hipErrorInvalidValue;
  }
  if (kv_fmt == kKvE4m3) return launch_tile_fmt<kKvE4m3, kQBf16>(p, tile_rows, gd, stream);
  if (kv_fmt == kKvE5m2) return launch_tile_fmt<kKvE5m2, kQBf16>(p, tile_rows, gd, stream);
  return launch_tile_fmt<kKvBf16, kQBf16>(p, tile_rows, gd, stream);
}

}  // namespace msa
