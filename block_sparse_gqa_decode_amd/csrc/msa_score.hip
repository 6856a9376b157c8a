// Indexer block-max scorer and top-k block selector for gfx950.
//
// Scorer: score[h, b, t] = max over the group's q heads g and the keys i of
// block b visible at token t's position of q[t, h*G+g] . K[page(b), h, i],
// -inf for blocks that start after the position (TensorRT-LLM PR #17171
// "Custom decode kernels for MinimaxM3", indexer commit: per-block causal max
// of Q.K, here with the q heads as the 16 columns of the same S^T = K Q^T MFMA
// tile the attend uses).
//
// Formats as in the attend: K is bf16, e4m3fn, e5m2 or MXFP4; q is bf16 or fp8
// e4m3fn with a per-tensor q scale.  With an fp8 q each 16-key tile is one
// 16x16x128 fp8 MFMA on the K bytes as loaded; with a bf16 q the K bytes are
// widened to bf16 for the bf16 MFMA.  q_scale * k_scale multiplies every dot
// product before the max.
//
// Work decomposition.  The visible (kv head, request, block) items -- every
// block a request's last token can see -- are counted on the device from
// seq_lens (a prefix sum over the batch in LDS), and each workgroup of a
// persistent grid takes an equal contiguous slice of them.  A slice is walked
// as segments of consecutive blocks of one (request, kv head): per segment the
// q operand is loaded once and the blocks' K halves stream through a
// kScoreDepth-deep register ring, each of the 4 wavefronts reading 32 keys of
// every block (4 KiB), so loads stay deep without many registers.  Per-block
// wavefront maxima meet in LDS and are written every kFlush items.  Cells of
// blocks past a request's last block, and padding rows, get -inf in a separate
// strided pass of the same grid.
//
// Selector: per (token, kv head), the k blocks with score > -inf in
// (score descending, block ascending) order, padded with -1 (same PR, top-k
// selector; ties to the lower block index), by an exact radix select over
// order-preserving integer images of the scores.
#include <climits>

#include "msa_device.h"
#include "msa_internal.h"
#include "msa_page.h"
#include "msa_select.h"

namespace msa {
namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreThreads = 64 * kScoreWaves;
constexpr int kScoreKeys = 32;     // keys of a block per wavefront
constexpr int kScoreDepth = 3;     // blocks in flight per wavefront (4: +1.3 us on the
                                   // full indexer step, 5 / 6: +2 / +8 us)
constexpr int kFlush = 32;         // items between LDS flushes of the maxima

// The K halves of one block for one wavefront (its 32 keys), by KV kind; the
// members follow PageRegs so the page header's widening helpers apply.
template <int kKind>
struct KHalf;

template <>
struct KHalf<1> {
  u32x4_t k[2][2];  // [key tile][run of 16 fp8]
};

template <>
struct KHalf<0> {
  u32x4_t k[2][4];  // [key tile][chunk of 8 bf16]
};

template <>
struct KHalf<2> {
  u32x4_t k[2];     // [key tile]: 32 e2m1 codes, head dims 32g..32g+31
  uint32_t ks[2];   // [key tile]: the key row's four block-scale codes
};

// `row_stride`: byte stride of packed K|V rows (unused for a 4-bit K slot).
template <int kKind>
__device__ __forceinline__ void load_khalf(KHalf<kKind>& r, const uint8_t* page,
                                           uint32_t row_stride, int lim, int kbase, int n,
                                           int g) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint32_t row = (uint32_t)min(kbase + 16 * tau + n, lim);
    if constexpr (kKind == 2) {
      r.k[tau] = *reinterpret_cast<const u32x4_t*>(page + row * kF4RowBytes + 16u * g);
      r.ks[tau] = *reinterpret_cast<const uint32_t*>(page + kF4ScaleBase + row * 4u);
    } else {
      const uint32_t off = row * row_stride + (kKind == 1 ? 16u * g : 32u * g);
      if constexpr (kKind == 1) {
        r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(page + off);
        r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(page + off + 64);
      } else {
        r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(page + off);
        r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(page + off + 16);
        r.k[tau][2] = *reinterpret_cast<const u32x4_t*>(page + off + 128);
        r.k[tau][3] = *reinterpret_cast<const u32x4_t*>(page + off + 144);
      }
    }
  }
}

template <int kKind, int kQ>
__device__ __forceinline__ void load_q(QRegs<kQ>& qf, const ScoreParams& p, int t, int h,
                                       int n, int g) {
  const int64_t row = (int64_t)t * p.hq + h * p.group + n;
  load_q_operand<kKind, kQ>(qf, p.q + row * kHeadDim * (kQ == kQE4m3 ? 1 : 2), n < p.group,
                            g);
}

// The max over a wavefront's 64 lanes, returned to every lane.  DPP row
// shifts and row broadcasts (the GCN lane network CDNA keeps) take the max
// into lane 63 in seven steps with no LDS round trip; the lane shuffles this
// replaces went through LDS, six dependent round trips per block (full
// indexer step 348 -> 344 us).  Every lane must be active.
__device__ __forceinline__ float wave_max_dpp(float v) {
  const int ninf = __float_as_int(-INFINITY);
  // A lane whose source is outside its row, or in a row the step does not
  // write, keeps -inf, which leaves its max unchanged.
#define MSA_DPP_MAX(ctrl, row_mask, bank_mask)                                       \
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), ctrl, \
                                                          row_mask, bank_mask, false)))
  MSA_DPP_MAX(0x111, 0xf, 0xf);  // row_shr:1
  MSA_DPP_MAX(0x112, 0xf, 0xf);  // row_shr:2
  MSA_DPP_MAX(0x113, 0xf, 0xf);  // row_shr:3: lane i of a row holds lanes i-3..i
  MSA_DPP_MAX(0x114, 0xf, 0xe);  // row_shr:4 into lanes 4..15
  MSA_DPP_MAX(0x118, 0xf, 0xc);  // row_shr:8 into lanes 8..15: lane 15 holds its row
  MSA_DPP_MAX(0x142, 0xa, 0xf);  // row_bcast:15 into rows 1 and 3
  MSA_DPP_MAX(0x143, 0xc, 0xf);  // row_bcast:31 into rows 2 and 3: lane 63 holds all
#undef MSA_DPP_MAX
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The wavefront's max over its 32 keys (those < nvis) and the group's rows of
// qk_scale * q.k for one block and one token.
template <int kKv, int kQ>
__device__ __forceinline__ float block_max(const KHalf<kv_kind(kKv)>& r,
                                           const QRegs<kQ>& qf, int kbase, int nvis, int n,
                                           int g, int group, float qk_scale) {
  float best = -INFINITY;
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (kQ == kQE4m3) {
      s = score_tile_fp8q<kKv>(r, qf, tau, 8u * g);
    } else {
      bf16x8_t kf[4];
      widen_k_tile<kKv>(r, tau, 8u * g, kf);
#pragma unroll
      for (int c = 0; c < 4; ++c) s = mfma_bf16_16x16x32(kf[c], qf.f[c], s);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kbase + 16 * tau + 4 * g + i;
      if (key < nvis && n < group) best = fmaxf(best, s[i] * qk_scale);
    }
  }
  return wave_max_dpp(best);
}

typedef __attribute__((address_space(4))) const int32_t const_i32;

template <int kKv, int kQ, bool kOneToken>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreParams p) {
  constexpr int kKind = kv_kind(kKv);
  __shared__ int32_t s_pref[kMaxScoreBatch + 1];       // blocks before request r
  __shared__ int32_t s_scan[kScoreThreads];
  __shared__ float s_part[kScoreWaves][kFlush * kMaxScoreDql];
  __shared__ int32_t s_item_r[kFlush], s_item_h[kFlush], s_item_b[kFlush];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Prefix sum of visible blocks per request (a request's last token sees
  // blocks 0 .. (seq_len-1)/128, within the score buffer and the table row).
  if (tid == 0) s_pref[0] = 0;
  int carry = 0;
  for (int base = 0; base < p.batch; base += kScoreThreads) {
    const int r = base + tid;
    int nb = 0;
    if (r < p.batch) {
      const int s = p.seq_lens[r];
      nb = s > 0 ? min((s - 1) / kPage + 1, min(p.max_blocks, p.bt_stride)) : 0;
    }
    s_scan[tid] = nb;
    __syncthreads();
    for (int off = 1; off < kScoreThreads; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    if (r < p.batch) s_pref[r + 1] = carry + s_scan[tid];
    carry += s_scan[kScoreThreads - 1];
    __syncthreads();
  }
  // Values read from LDS are made wavefront-uniform (readfirstlane) so that
  // the walk below runs on scalar registers and its table reads are scalar.
  const int per_head = __builtin_amdgcn_readfirstlane(s_pref[p.batch]);
  const int64_t total = (int64_t)per_head * p.hkv;

  // -inf for cells of blocks past a request's last block and for padding rows,
  // visited with the smaller of the block and token strides innermost so the
  // stores coalesce for either buffer orientation.
  {
    const int64_t cells = (int64_t)p.hkv * p.max_blocks * p.num_rows;
    const bool b_inner = p.sc_s1 < p.sc_s2;
    const int inner = b_inner ? p.max_blocks : p.num_rows;
    const int outer = b_inner ? p.num_rows : p.max_blocks;
    for (int64_t c = (int64_t)blockIdx.x * kScoreThreads + tid; c < cells;
         c += (int64_t)gridDim.x * kScoreThreads) {
      const int i_in = (int)(c % inner);
      const int64_t rest = c / inner;
      const int i_out = (int)(rest % outer);
      const int h = (int)(rest / outer);
      const int b = b_inner ? i_in : i_out;
      const int t = b_inner ? i_out : i_in;
      bool dead = t >= p.real_rows;
      if (!dead) {
        const int r = t / p.dql;
        dead = b >= s_pref[r + 1] - s_pref[r];
      }
      if (dead) p.score[h * p.sc_s0 + (int64_t)b * p.sc_s1 + (int64_t)t * p.sc_s2] = -INFINITY;
    }
  }

  // This workgroup's slice of the visible items [i0, i1).
  const int64_t i0 = total * blockIdx.x / gridDim.x;
  const int64_t i1 = total * (blockIdx.x + 1) / gridDim.x;
  if (i0 >= i1) return;

  const int kbase = wave * kScoreKeys;
  const uint32_t row_stride = (uint32_t)p.kv_s2;
  int nflush = 0;

  // Walk the slice as segments of one (kv head, request).
  int64_t item = i0;
  int h = (int)(item / per_head);
  int rem = (int)(item - (int64_t)h * per_head);
  int r = 0;
  {  // first request with s_pref[r+1] > rem
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid + 1] > rem) hi = mid; else lo = mid + 1;
    }
    r = __builtin_amdgcn_readfirstlane(lo);
  }
  int b = __builtin_amdgcn_readfirstlane(rem - s_pref[r]);

  while (item < i1) {
    r = __builtin_amdgcn_readfirstlane(r);
    b = __builtin_amdgcn_readfirstlane(b);
    h = __builtin_amdgcn_readfirstlane(h);
    const int nb_r = __builtin_amdgcn_readfirstlane(s_pref[r + 1] - s_pref[r]);
    const int seg = (int)min((int64_t)(nb_r - b), i1 - item);
    const int seq = ((const const_i32*)p.seq_lens)[r];
    const int t0 = r * p.dql;
    const int32_t* bt_row = p.block_table + (int64_t)r * p.bt_stride;
    const uint8_t* head_base = p.kv + h * p.kv_s1;
    QRegs<kQ> qf;
    load_q<kKind, kQ>(qf, p, t0 + p.dql - 1, h, n, g);
    const int b_last = b + seg - 1;

    // Block-table entries are read through the scalar cache (uniform index,
    // constant address space), so no vector load sits in the ring.
    const const_i32* bt_c = (const const_i32*)(bt_row);
    auto page_of = [&](int bb, int& lim) -> const uint8_t* {
      int pg = bt_c[__builtin_amdgcn_readfirstlane(bb)];
      if (pg < 0 || pg >= p.num_kv_blocks) pg = -1;
      const int nvis = min(kPage, seq - 1 - bb * kPage + 1);
      lim = nvis - 1;
      return pg < 0 ? nullptr : head_base + (int64_t)pg * p.kv_s0;
    };

    KHalf<kKind> buf[kScoreDepth];
    const uint8_t* pages[kScoreDepth];
    int lims[kScoreDepth];
#pragma unroll
    for (int j = 0; j < kScoreDepth - 1; ++j) {
      const int bb = min(b + j, b_last);
      pages[j] = page_of(bb, lims[j]);
      load_khalf<kKind>(buf[j], pages[j] ? pages[j] : head_base, row_stride,
                        pages[j] ? lims[j] : 0, kbase, n, g);
    }
    for (int i = 0;; i += kScoreDepth) {
#pragma unroll
      for (int j = 0; j < kScoreDepth; ++j) {
        if (i + j >= seg) goto segment_done;
        {
          const int jn = (j + kScoreDepth - 1) % kScoreDepth;
          const int bn = min(b + i + j + kScoreDepth - 1, b_last);
          pages[jn] = page_of(bn, lims[jn]);
          load_khalf<kKind>(buf[jn], pages[jn] ? pages[jn] : head_base, row_stride,
                            pages[jn] ? lims[jn] : 0, kbase, n, g);
          const int bb = b + i + j;
          const bool ok_page = pages[j] != nullptr;
          // token loop: the last token sees the most; earlier tokens fewer keys
          for (int l = 0; l < p.dql; ++l) {
            const int pos = seq - p.dql + l;
            const int nvis = pos - bb * kPage + 1;
            float m = -INFINITY;
            if (ok_page && nvis > 0 && kbase < nvis) {
              if constexpr (kOneToken) {
                m = block_max<kKv, kQ>(buf[j], qf, kbase, min(nvis, kPage), n, g, p.group,
                                       p.qk_scale);
              } else {
                QRegs<kQ> ql;
                load_q<kKind, kQ>(ql, p, t0 + l, h, n, g);
                m = block_max<kKv, kQ>(buf[j], ql, kbase, min(nvis, kPage), n, g, p.group,
                                       p.qk_scale);
              }
            }
            if (lane == 0) s_part[wave][nflush * p.dql + l] = m;
          }
          if (tid == 0) {
            s_item_r[nflush] = r;
            s_item_h[nflush] = h;
            s_item_b[nflush] = bb;
          }
          ++nflush;
          if (nflush == kFlush) {
            __syncthreads();
            for (int e = tid; e < kFlush * p.dql; e += kScoreThreads) {
              const int it = e / p.dql, l = e - it * p.dql;
              float m = s_part[0][e];
#pragma unroll
              for (int w = 1; w < kScoreWaves; ++w) m = fmaxf(m, s_part[w][e]);
              p.score[s_item_h[it] * p.sc_s0 + (int64_t)s_item_b[it] * p.sc_s1 +
                      (int64_t)(s_item_r[it] * p.dql + l) * p.sc_s2] = m;
            }
            __syncthreads();
            nflush = 0;
          }
        }
      }
    }
  segment_done:
    item += seg;
    b += seg;
    if (b >= nb_r) {  // next request (skipping empty ones), then next head
      b = 0;
      do {
        if (++r == p.batch) {
          r = 0;
          ++h;
        }
      } while (item < i1 && __builtin_amdgcn_readfirstlane(s_pref[r + 1] - s_pref[r]) == 0);
    }
  }
  __syncthreads();
  for (int e = tid; e < nflush * p.dql; e += kScoreThreads) {
    const int it = e / p.dql, l = e - it * p.dql;
    float m = s_part[0][e];
#pragma unroll
    for (int w = 1; w < kScoreWaves; ++w) m = fmaxf(m, s_part[w][e]);
    p.score[s_item_h[it] * p.sc_s0 + (int64_t)s_item_b[it] * p.sc_s1 +
            (int64_t)(s_item_r[it] * p.dql + l) * p.sc_s2] = m;
  }
}

// One workgroup per (token row, kv head); the selection itself is select_row
// (msa_select.h), shared with the attend that selects its own pages.
template <int kPer>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  __shared__ SelShared sh;
  const int t = blockIdx.x / p.hkv;
  const int h = blockIdx.x - t * p.hkv;
  select_row<kPer>(p.score + h * p.sc_s0 + (int64_t)t * p.sc_s2, p.sc_s1, p.max_blocks, p.k,
                   sh, p.topk_out + ((int64_t)t * p.hkv + h) * p.k);
}
}  // namespace

template <int kKv, int kQ>
static void launch_score_fmt(const ScoreParams& p, dim3 g, dim3 b, hipStream_t stream) {
  if (p.dql == 1) hipLaunchKernelGGL((score_kernel<kKv, kQ, true>), g, b, 0, stream, p);
  else hipLaunchKernelGGL((score_kernel<kKv, kQ, false>), g, b, 0, stream, p);
}

hipError_t launch_score(const ScoreParams& p, int kv_fmt, int q_fmt, hipStream_t stream) {
  // A persistent grid: three workgroups per CU (measured on the full decode
  // step: 768 beats 512 and 1024 by 1-2%, 256 / 384 lose 5-7%), never more
  // than there are possible items.
  const int64_t upper = (int64_t)p.batch * p.hkv * p.max_blocks;
  const int64_t grid = upper < 768 ? (upper > 0 ? upper : 1) : 768;
  const dim3 g((uint32_t)grid), b(kScoreThreads);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3) launch_score_fmt<kKvE4m3, kQE4m3>(p, g, b, stream);
    else if (kv_fmt == kKvE5m2) launch_score_fmt<kKvE5m2, kQE4m3>(p, g, b, stream);
    else if (kv_fmt == kKvMxfp4) launch_score_fmt<kKvMxfp4, kQE4m3>(p, g, b, stream);
    else return hipErrorInvalidValue;
  } else {
    if (kv_fmt == kKvE4m3) launch_score_fmt<kKvE4m3, kQBf16>(p, g, b, stream);
    else if (kv_fmt == kKvE5m2) launch_score_fmt<kKvE5m2, kQBf16>(p, g, b, stream);
    else if (kv_fmt == kKvMxfp4) launch_score_fmt<kKvMxfp4, kQBf16>(p, g, b, stream);
    else launch_score_fmt<kKvBf16, kQBf16>(p, g, b, stream);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_rows * p.hkv;
  if (grid <= 0) return hipSuccess;
  const dim3 g((uint32_t)grid), b(kSelThreads);
  const int per = (p.max_blocks + kSelThreads - 1) / kSelThreads;
  if (per <= 2) hipLaunchKernelGGL((select_kernel<2>), g, b, 0, stream, p);
  else if (per <= 8) hipLaunchKernelGGL((select_kernel<8>), g, b, 0, stream, p);
  else if (per <= 32) hipLaunchKernelGGL((select_kernel<32>), g, b, 0, stream, p);
  else hipLaunchKernelGGL((select_kernel<64>), g, b, 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
