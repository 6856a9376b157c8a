// Per-page machinery of the attend kernels for gfx950: the register ring of
// one wavefront's 32 keys of a KV page, their loads, the S^T tile and the
// whole per-page step (mask, online softmax, P V).
//
// Register layouts (16x16x32 bf16 MFMA, lane l, n = l % 16, g = l / 16):
//  * S^T = K Q^T: A = K rows (key n of a 16-key tile), B = Q^T (q row n).  The
//    contraction slot (g, c, j) of chunk c maps to head dim
//    d = 64*(c/2) + 16*g + 8*(c%2) + j, so a lane reads two contiguous 16-dim
//    runs of its key row.  The accumulator gives lane l the scores of keys
//    4g..4g+3 of the tile for q row n.  With an fp8 q the tile is one
//    16x16x128 fp8 MFMA on the same two runs.
//  * O^T += V^T P^T: B = P^T comes straight from the two S^T accumulators of
//    the wavefront's 32 keys (contraction slot j of group g = key 4g+j for
//    j<4, 16+4g+(j-4) for j>=4).  A = V^T uses the same key slots; its row m
//    of d-tile t8 is head dim 8m+t8, so lane l loads the 8 contiguous head
//    dims 8n..8n+7 of each of its 8 keys and a byte permute transposes them
//    into the 8 d-tiles.  The accumulator then holds O[q row n][32g + 8i + t8]
//    for i < 4, t8 < 8: 32 contiguous outputs.
#pragma once

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

constexpr int kWaves = 4;      // wavefronts sharing one page (32 keys each)
constexpr int kThreads = 64 * kWaves;
constexpr int kDepth = 2;      // pages per wavefront in the register ring
constexpr int kTableLoads = 8; // block-table entries per thread read ahead (2048 a workgroup)

constexpr int kKeysPerWave = 32;
constexpr int kOPad = 4;
constexpr float kRescaleSlack = 8.0f;

// KV element kinds: 0 = 16-bit (bf16), 1 = 8-bit (fp8 e4m3fn / e5m2),
// 2 = 4-bit (MXFP4 head slots).
constexpr int kv_kind(int kKv) { return kKv == kKvBf16 ? 0 : (kKv == kKvMxfp4 ? 2 : 1); }

template <int kKind>
struct PageRegs;

template <>
struct PageRegs<1> {
  u32x4_t k[2][2];  // [key tile][run]: 16 fp8 each (head dims 16g.., 64+16g..)
  u32x2_t v[8];     // 8 fp8 (head dims 8n..8n+7) of key slot j
};

template <>
struct PageRegs<0> {
  u32x4_t k[2][4];  // [key tile][chunk]: 8 bf16 each
  u32x4_t v[8];     // 8 bf16 of key slot j
};

template <>
struct PageRegs<2> {
  u32x4_t k[2];     // [key tile]: 32 e2m1 codes, head dims 32g..32g+31
  uint32_t ks[2];   // [key tile]: the key row's four K block-scale codes
  uint32_t v[8];    // 8 e2m1 codes (head dims 8n..8n+7) of key slot j
  uint32_t vs[8];   // key slot j's four V block-scale codes
};

__device__ __forceinline__ int key_of_slot(int g, int j) {
  return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// Per-lane constants of the page loads: the page rows a lane reads for the two
// S^T tiles and the eight P^T / V^T slots, its byte columns, and (4-bit pages)
// the bit offsets of its K and V block scales within a row's scale dword.
struct LaneRows {
  int rk[2];
  int rv[8];
  uint32_t ck;  // first K byte of the lane's runs
  uint32_t cv;  // first V byte of the lane's run
  uint32_t ksh; // 8 * (K block of head dims 32g..32g+31) = 8g
  uint32_t vsh; // 8 * (V block of head dims 8n..8n+7) = 8 * (n / 4)
  // 16- and 8-bit pages: the byte offsets of the lane's K runs and V runs
  // within a page-head, row * row_stride + column (set by lane_offsets).
  uint32_t ok[2];
  uint32_t ov[8];
};

// kWholeK (8-bit K, the row-tile kernels): each K load reads 8 whole rows,
// lane 16g + n taking row 2g + n / 8 of the 8 and bytes 16 (n % 8) .. +15,
// the second load the next 8 rows; k8_whole_to_mfma then moves the bytes
// into the MFMA's layout.
template <int kKind, bool kWholeK = false>
__device__ __forceinline__ LaneRows lane_rows(int kbase, int n, int g) {
  LaneRows lr;
  constexpr bool kWhole = kWholeK && kKind == 1;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau)
    lr.rk[tau] = kbase + 16 * tau + (kWhole ? 2 * g + (n >> 3) : n);
#pragma unroll
  for (int j = 0; j < 8; ++j) lr.rv[j] = kbase + key_of_slot(g, j);
  lr.ck = kKind == 0 ? 32u * g : (kWhole ? 16u * (uint32_t)(n & 7) : 16u * g);
  lr.cv = kKind == 0 ? 2 * kHeadDim + 16u * n : (kKind == 1 ? kHeadDim + 8u * n : 4u * n);
  lr.ksh = 8u * g;
  lr.vsh = 8u * (n >> 2);
  return lr;
}

// The per-lane byte offsets of the 16- and 8-bit page loads, fixed for a
// launch (row strides < 2^24, so 24-bit multiplies).
__device__ __forceinline__ void lane_offsets(LaneRows& lr, uint32_t row_stride) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) lr.ok[tau] = __umul24((uint32_t)lr.rk[tau], row_stride) + lr.ck;
#pragma unroll
  for (int j = 0; j < 8; ++j) lr.ov[j] = __umul24((uint32_t)lr.rv[j], row_stride) + lr.cv;
}

// 4-bit head slot: 128 rows x 64 data bytes, then 128 rows x 4 scale bytes.
constexpr uint32_t kF4RowBytes = kHeadDim / 2;
constexpr uint32_t kF4ScaleBase = kPage * kF4RowBytes;

// Loads of one page into registers.  `page` is wave-uniform (SGPRs); rows are
// clamped to the last visible row `lim`, so rows past it are never read; the
// per-lane part of every address is a 32-bit offset.  `row_stride` is the
// byte stride of packed K|V rows, or for 4-bit pages the K slot -> V slot
// offset.
template <int kKind, bool kWholeK = false>
__device__ __forceinline__ void load_page(PageRegs<kKind>& r, const uint8_t* page,
                                          uint32_t row_stride, int lim, const LaneRows& lr) {
  if constexpr (kKind == 2) {
    const uint8_t* vpage = page + row_stride;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const uint32_t row = (uint32_t)min(lr.rk[tau], lim);
      r.k[tau] = *reinterpret_cast<const u32x4_t*>(page + row * kF4RowBytes + lr.ck);
      r.ks[tau] = *reinterpret_cast<const uint32_t*>(page + kF4ScaleBase + row * 4u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t row = (uint32_t)min(lr.rv[j], lim);
      r.v[j] = *reinterpret_cast<const uint32_t*>(vpage + row * kF4RowBytes + lr.cv);
      r.vs[j] = *reinterpret_cast<const uint32_t*>(vpage + kF4ScaleBase + row * 4u);
    }
    return;
  } else {
    // Row offsets by 24-bit multiplies (rows < 128, row strides < 2^24).
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const uint32_t off = __umul24((uint32_t)min(lr.rk[tau], lim), row_stride) + lr.ck;
      if constexpr (kKind == 1 && kWholeK) {
        const uint32_t off8 = __umul24((uint32_t)min(lr.rk[tau] + 8, lim), row_stride) + lr.ck;
        r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(page + off);
        r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(page + off8);
      } else if constexpr (kKind == 1) {
        r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(page + off);
        r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(page + off + 64);
      } else {
        r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(page + off);
        r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(page + off + 16);
        r.k[tau][2] = *reinterpret_cast<const u32x4_t*>(page + off + 128);
        r.k[tau][3] = *reinterpret_cast<const u32x4_t*>(page + off + 144);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = __umul24((uint32_t)min(lr.rv[j], lim), row_stride) + lr.cv;
      if constexpr (kKind == 1) {
        r.v[j] = *reinterpret_cast<const u32x2_t*>(page + off);
      } else {
        r.v[j] = *reinterpret_cast<const u32x4_t*>(page + off);
      }
    }
  }
}

constexpr int kRsrcWord3 = 0x00020000;    // raw buffer descriptor, gfx9 family

// Loads of one page into registers through a buffer descriptor whose size is
// the page-head's first `nvis` rows: the hardware returns zeros for every
// lane whose row is past them, so stale rows are never read and no lane
// offset is recomputed per page (16- and 8-bit pages; offsets from
// lane_offsets).  4-bit pages, whose data and scales are separate runs, take
// the clamped loads of load_page.
template <int kKind, bool kWholeK = false>
__device__ __forceinline__ void load_page_rows(PageRegs<kKind>& r, const uint8_t* page,
                                               uint32_t row_stride, int nvis,
                                               const LaneRows& lr) {
  if constexpr (kKind == 2) {
    load_page<2>(r, page, row_stride, max(nvis, 1) - 1, lr);
  } else {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(page), (short)0, (int)((uint32_t)nvis * row_stride), kRsrcWord3);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      if constexpr (kKind == 1) {
        r.k[tau][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rs, lr.ok[tau], 0, 0));
        r.k[tau][1] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rs, kWholeK ? lr.ok[tau] + 8u * row_stride : lr.ok[tau] + 64u, 0, 0));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          r.k[tau][c] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, lr.ok[tau] + 16 * (c & 1) + 128 * (c >> 1), 0, 0));
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (kKind == 1)
        r.v[j] = __builtin_bit_cast(u32x2_t,
                                    __builtin_amdgcn_raw_buffer_load_b64(rs, lr.ov[j], 0, 0));
      else
        r.v[j] = __builtin_bit_cast(u32x4_t,
                                    __builtin_amdgcn_raw_buffer_load_b128(rs, lr.ov[j], 0, 0));
    }
  }
}

// A wavefront's whole-row 8-bit K registers (kWholeK loads) put into the
// MFMA's layout, lane 16g + n holding row n's bytes 16g.. and 64+16g.. of
// each key tile, through `scratch`, 4 KB of LDS the wavefront owns for the
// page loop.  Row r of a key tile is stored with 16-byte chunk c at position
// c ^ (r / 2 % 8): the writes (8 lanes a row) and the reads (16 rows, one
// chunk each) are then free of bank conflicts.  A wavefront's LDS accesses
// run in order, so the reads follow its own writes without a wait.
//
// Whole-row loads touch 8 full 128-byte lines each, where a load in the
// MFMA's layout (16 rows, 64 bytes of each, four lanes a row 64 bytes apart)
// touches 16 half lines and no two neighbouring lanes share a row.
__device__ __forceinline__ void k8_whole_to_mfma(PageRegs<1>& r, uint8_t* scratch, int n,
                                                 int g) {
  const int ln = 16 * g + n;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t row = 8u * h + (uint32_t)(ln >> 3);
      const uint32_t pos = (uint32_t)(ln & 7) ^ ((row >> 1) & 7u);
      *reinterpret_cast<u32x4_t*>(scratch + 2048u * tau + 128u * row + 16u * pos) = r.k[tau][h];
    }
  }
  const uint32_t f = ((uint32_t)n >> 1) & 7u;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint8_t* row = scratch + 2048u * tau + 128u * (uint32_t)n;
    r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(row + 16u * ((uint32_t)g ^ f));
    r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(row + 16u * ((4u + (uint32_t)g) ^ f));
  }
}

// The Q^T operand of q row `qp` (bytes; `load` false gives zeros).  A bf16 q
// takes the contraction slots the widened K of the KV kind holds: chunk c of
// lane group g is head dims 64*(c/2) + 16g + 8*(c%2) .. +7 (16/8-bit K), or
// 32g + 8c .. +7 (4-bit K, the lane's MX block).  An fp8 q takes the fp8
// MFMA's own layout, head dims 16g.. and 64+16g.. (both K kinds meet it).
template <int kKind, int kQ>
__device__ __forceinline__ void load_q_operand(QRegs<kQ>& qf, const uint8_t* qp, bool load,
                                               int g) {
  if constexpr (kQ == kQE4m3) {
    u32x4_t lo = u32x4_t{0u, 0u, 0u, 0u}, hi = lo;
    if (load) {
      lo = *reinterpret_cast<const u32x4_t*>(qp + 16 * g);
      hi = *reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g);
    }
    qf.b = cat_i32x8(lo, hi);
  } else {
    if (load) {
      const uint16_t* q16 = reinterpret_cast<const uint16_t*>(qp);
      if constexpr (kKind == 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          qf.f[c] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q16 + 32 * g + 8 * c));
      } else {
        qf.f[0] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q16 + 16 * g));
        qf.f[1] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q16 + 16 * g + 8));
        qf.f[2] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q16 + 64 + 16 * g));
        qf.f[3] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(q16 + 64 + 16 * g + 8));
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qf.f[c] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
    }
  }
}

// K tile tau widened to the four bf16 operand chunks of the bf16 MFMA.  `R`
// is any register set with the K members of PageRegs<kv_kind(kKv)>.
template <int kKv, class R>
__device__ __forceinline__ void widen_k_tile(const R& r, int tau, uint32_t ksh,
                                             bf16x8_t (&kf)[4]) {
  if constexpr (kv_kind(kKv) == 2) {
    const float sc = e8m0_scale_of(r.ks[tau], ksh);
    kf[0] = as_bf16x8(f4x8_to_bf16x8(r.k[tau].x, sc));
    kf[1] = as_bf16x8(f4x8_to_bf16x8(r.k[tau].y, sc));
    kf[2] = as_bf16x8(f4x8_to_bf16x8(r.k[tau].z, sc));
    kf[3] = as_bf16x8(f4x8_to_bf16x8(r.k[tau].w, sc));
  } else if constexpr (kv_kind(kKv) == 1) {
    kf[0] = as_bf16x8(f8x8_to_bf16x8<kKv>(r.k[tau][0].x, r.k[tau][0].y));
    kf[1] = as_bf16x8(f8x8_to_bf16x8<kKv>(r.k[tau][0].z, r.k[tau][0].w));
    kf[2] = as_bf16x8(f8x8_to_bf16x8<kKv>(r.k[tau][1].x, r.k[tau][1].y));
    kf[3] = as_bf16x8(f8x8_to_bf16x8<kKv>(r.k[tau][1].z, r.k[tau][1].w));
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[c] = as_bf16x8(r.k[tau][c]);
  }
}

// S^T tile tau with an fp8 q: one 16x16x128 MFMA on the K codes as loaded.
template <int kKv, class R>
__device__ __forceinline__ f32x4_t score_tile_fp8q(const R& r, const QRegs<kQE4m3>& q,
                                                   int tau, uint32_t ksh) {
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kv_kind(kKv) == 2) {
    return mfma_f4f8_16x16x128(r.k[tau], (int)((r.ks[tau] >> ksh) & 0xffu), q.b, zero);
  } else {
    return mfma_f8_16x16x128<kKv == kKvE5m2 ? 1 : 0, 0>(cat_i32x8(r.k[tau][0], r.k[tau][1]),
                                                         q.b, zero);
  }
}

// V rows of the eight key slots as bf16 pairs along the head dim:
// vd[j][w] = dims (8n+2w, 8n+2w+1) of key slot j.
template <int kKv>
__device__ __forceinline__ void widen_v(const PageRegs<kv_kind(kKv)>& r, uint32_t vsh,
                                        u32x4_t (&vd)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (kv_kind(kKv) == 2) {
      vd[j] = f4x8_to_bf16x8(r.v[j], e8m0_scale_of(r.vs[j], vsh));
    } else if constexpr (kv_kind(kKv) == 1) {
      vd[j] = f8x8_to_bf16x8<kKv>(r.v[j].x, r.v[j].y);
    } else {
      vd[j] = r.v[j];
    }
  }
}

// The eight V^T A operands of O^T += V^T P^T: vt[t8] holds, for head dim
// 8n + t8, the bf16 values of the lane's eight key slots in pairs
// (slot 2i, slot 2i+1) = dword i.  8-bit V: one byte permute gathers the two
// slots' bytes of dims t8 and t8+1, and the two halves of that dword convert
// straight into dword i of d-tiles t8 and t8+1 (16 permutes, 32 conversions).
// Other kinds widen each slot's eight dims first (per-key block scales for
// 4-bit V) and then transpose the bf16 pairs (32 permutes).
template <int kKv>
__device__ __forceinline__ void build_vt(const PageRegs<kv_kind(kKv)>& r, uint32_t vsh,
                                         u32x4_t (&vt)[8]) {
  if constexpr (kv_kind(kKv) == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = h ? r.v[2 * i].y : r.v[2 * i].x;
        const uint32_t hi = h ? r.v[2 * i + 1].y : r.v[2 * i + 1].x;
#pragma unroll
        for (int b = 0; b < 4; b += 2) {
          // bytes: slot 2i dim b, slot 2i+1 dim b, slot 2i dim b+1, slot 2i+1 dim b+1
          const uint32_t w = byte_perm(hi, lo, b == 0 ? 0x05010400u : 0x07030602u);
          const int t8 = 4 * h + b;
          if constexpr (kKv == kKvE5m2) {
            vt[t8][i] = bf8x2_to_bf16x2<false>(w);
            vt[t8 + 1][i] = bf8x2_to_bf16x2<true>(w);
          } else {
            vt[t8][i] = fp8x2_to_bf16x2<false>(w);
            vt[t8 + 1][i] = fp8x2_to_bf16x2<true>(w);
          }
        }
      }
    }
  } else {
    u32x4_t vd[8];
    widen_v<kKv>(r, vsh, vd);
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
      const uint32_t sel = (t8 & 1) ? 0x07060302u : 0x05040100u;
      const int w = t8 >> 1;
      vt[t8].x = byte_perm(vd[1][w], vd[0][w], sel);
      vt[t8].y = byte_perm(vd[3][w], vd[2][w], sel);
      vt[t8].z = byte_perm(vd[5][w], vd[4][w], sel);
      vt[t8].w = byte_perm(vd[7][w], vd[6][w], sel);
    }
  }
}

// S^T tile tau (16 keys x 16 q rows) of one page.
template <int kKv, int kQ>
__device__ __forceinline__ f32x4_t score_tile(const PageRegs<kv_kind(kKv)>& r,
                                              const QRegs<kQ>& q, int tau, uint32_t ksh) {
  if constexpr (kQ == kQE4m3) {
    return score_tile_fp8q<kKv>(r, q, tau, ksh);
  } else {
    bf16x8_t kf[4];
    widen_k_tile<kKv>(r, tau, ksh, kf);
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma_bf16_16x16x32(kf[c], q.f[c], s);
    return s;
  }
}

// One page of the online softmax for the lane's eight scores z (raw S^T
// values, -inf where masked) of q row n: the probabilities
// 2^(z * scale_log2 - m_run) as the bf16 P^T operand, with l_part and the O
// accumulators kept consistent with the reference point m_run.
//
// Lazy rescaling: a row's reference only moves when its probabilities would
// grow too large.  The test is on the sum of the lane's eight probabilities,
// which the step needs anyway: while every lane's sum stays <= 8 * 2^kRescaleSlack
// (so each probability is bounded), nothing else is computed.  Otherwise (a
// score more than about kRescaleSlack above the reference, or the row's first
// keys with m_run = -inf, which gives inf / NaN sums) the wave forms the row
// maxima, moves the reference of every row whose maximum exceeds it by more
// than kRescaleSlack, rescales O and l and recomputes the probabilities.
__device__ __forceinline__ bf16x8_t softmax_step(const float (&z)[8], float scale_log2,
                                                 float& m_run, float& l_part,
                                                 f32x4_t (&o)[8]) {
  constexpr float kLaneSumCap = 8.0f * 256.0f;  // 8 * 2^kRescaleSlack
  float pz[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pz[e] = fast_exp2(fmaf(z[e], scale_log2, -m_run));
  float ls = ((pz[0] + pz[1]) + (pz[2] + pz[3])) + ((pz[4] + pz[5]) + (pz[6] + pz[7]));
  if (__any(!(ls <= kLaneSumCap))) {
    const float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                           fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7]))) * scale_log2;
    const float mrow = wave_max_xor_16_32(mx);
    if (mrow > m_run + kRescaleSlack) {
      const float alpha = fast_exp2(m_run - mrow);
      l_part *= alpha;
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) o[t8] *= alpha;
      m_run = mrow;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pz[e] = fast_exp2(fmaf(z[e], scale_log2, -m_run));
    ls = ((pz[0] + pz[1]) + (pz[2] + pz[3])) + ((pz[4] + pz[5]) + (pz[6] + pz[7]));
  }
  l_part += ls;
  u32x4_t pw;
  pw.x = pack_bf16x2(pz[0], pz[1]);
  pw.y = pack_bf16x2(pz[2], pz[3]);
  pw.z = pack_bf16x2(pz[4], pz[5]);
  pw.w = pack_bf16x2(pz[6], pz[7]);
  return as_bf16x8(pw);
}

template <int kKv, int kQ>
__device__ __forceinline__ void attend_page(const PageRegs<kv_kind(kKv)>& r,
                                            const QRegs<kQ>& qf, const LaneRows& lr,
                                            int kbase, int nvis, int g, float scale_log2,
                                            float& m_run, float& l_part,
                                            f32x4_t (&o)[8]) {
  // S^T for the wavefront's two 16-key tiles.
  f32x4_t s[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) s[tau] = score_tile<kKv, kQ>(r, qf, tau, lr.ksh);

  // Raw scores; keys past the visible count (only on a token's last page)
  // become -inf.  The softmax step applies the positive scale.
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
      for (int i = 0; i < 4; ++i) {
        if (kbase + 16 * tau + 4 * g + i >= nvis) z[4 * tau + i] = -INFINITY;
      }
    }
  }
  const bf16x8_t pb = softmax_step(z, scale_log2, m_run, l_part, o);

  u32x4_t vt[8];
  build_vt<kKv>(r, lr.vsh, vt);
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) o[t8] = mfma_bf16_16x16x32(as_bf16x8(vt[t8]), pb, o[t8]);
}

// bf16 store of one output row chunk: acc / L * v_scale, or exact zeros when
// the row saw no key (L == 0).  A NaN sum (a NaN logit from NaN cache
// entries) is stored as NaN, as the definition gives, not as an empty row.
// Branch-free (selects, not a branch), so a caller's loads that feed acc are
// not sunk behind the test of L and stay issued together.
__device__ __forceinline__ void store_row(uint16_t* dst, const float (&acc)[8], float L,
                                          float v_scale) {
  const bool live = L != 0.f;
  const float inv = live ? v_scale / L : 0.f;
  u32x4_t ov;
  ov.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  ov.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  ov.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  ov.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  ov.x = live ? ov.x : 0u;
  ov.y = live ? ov.y : 0u;
  ov.z = live ? ov.z : 0u;
  ov.w = live ? ov.w : 0u;
  *reinterpret_cast<u32x4_t*>(dst) = ov;
}

}  // namespace msa
