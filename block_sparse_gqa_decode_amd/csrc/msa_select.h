// Exact top-k block selection over one row of block scores, shared by the
// selector kernel (msa_score.hip) and the attend that selects its own pages
// (msa_attend.hip).
//
// Per (token, kv head) row: the k blocks with score > -inf in (score
// descending, block ascending) order, padded with -1 (TensorRT-LLM PR #17171,
// indexer-scorer commit: the top-k selector after the per-block max; ties to
// the lower block index), by an exact prefilter and, when ties crowd it, a
// radix select over order-preserving integer images of the scores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_internal.h"

namespace msa {

constexpr int kSelThreads = 256;

// Order-preserving unsigned image of a score: larger score -> larger key.
// -inf and NaN map to 0 (never selected); -0 maps like +0 so that the two rank
// as equal, as they compare.
__device__ __forceinline__ uint32_t order_key(float v) {
  if (!(v > -INFINITY)) return 0u;
  uint32_t u = __float_as_uint(v);
  if (v == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wavefront 0 of a radix-select pass: hist holds 256 digit counts; finds the
// digit d such that the `need`-th largest counted element has digit d.
// ctl[0] = d, ctl[1] = elements still needed inside bin d, ctl[2] = count of
// bin d, ctl[3] = total counted.  Writes ctl[0..2] only if total >= need.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, int lane, uint32_t need,
                                           uint32_t* ctl) {
  uint32_t h[4];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = hist[4 * lane + i];
    sum += h[i];
  }
  uint32_t suffix = sum;  // count in this lane's bins and every higher bin
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(suffix, off);
    if (lane + off < 64) suffix += v;
  }
  const uint32_t above = suffix - sum;
  if (suffix >= need && above < need) {
    uint32_t acc = above;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (acc + h[i] >= need) {
        ctl[0] = 4 * lane + i;
        ctl[1] = need - acc;
        ctl[2] = h[i];
        break;
      }
      acc += h[i];
    }
  }
  if (lane == 0) ctl[3] = suffix;
}

// One workgroup per (token row, kv head).  The row's scores live in registers
// (kPer per thread, block b = tid + 256 i).
//
// Prefilter, exact: let T0 be the k-th largest of the 256 per-thread maxima
// (0 when fewer than k threads hold a selectable key).  The k maxima ranked
// at or above it are k distinct keys >= T0, so the k-th largest key of the
// row is >= T0 and every block the selection keeps (ties at the k-th key
// included) has a key >= T0.  Wavefront 0 finds T0 bit by bit with ballot
// counts; the blocks with keys >= T0 (about k of them on unequal scores, at
// most kPer * k when the maxima are distinct) are compacted into LDS and each
// is ranked by (key desc, block asc) with one 64-bit comparison per pair.
//
// If ties leave more than kSelCap candidates, a most-significant-digit radix
// select over all keys (four 8-bit passes with LDS histograms) finds the k-th
// largest key T exactly; if only some of the blocks whose key equals T fit,
// two 7-bit passes over (16383 - block) pick the lowest block ids among them.
// The at most k chosen blocks are then ranked as above.
constexpr int kSelCap = 512;

// (key desc, block asc) as one unsigned order: the key above the inverted
// 14-bit block id, so a larger packed value ranks first.
__device__ __forceinline__ uint64_t pack_rank_key(uint32_t key, int block) {
  return ((uint64_t)key << 14) | (uint64_t)(kMaxScoreBlocks - 1 - block);
}


// LDS of one selection (a workgroup of kSelThreads threads).
struct SelShared {
  uint32_t max[kSelThreads];
  uint32_t t0;
  uint32_t wcnt[kSelThreads / 64];
  uint64_t cand[kSelCap];
  uint32_t hist[256];
  uint32_t ctl[4];
  uint32_t nsel;
  uint32_t sel_key[kMaxTopk];
  int32_t sel_blk[kMaxTopk];
};

// The selection of one row by a workgroup of exactly kSelThreads threads
// (all of them call it): srow[b * sc_s1] for b < nblk (kPer * kSelThreads >=
// nblk) are the row's scores; out[0..kk) receives the blocks in rank order
// and -1 padding (out may be LDS or global memory).  The caller synchronizes
// before reading an LDS out.
template <int kPer>
__device__ __forceinline__ void select_row(const float* srow, int64_t sc_s1, int nblk, int kk,
                                           SelShared& sh, int32_t* out) {
  uint32_t* s_max = sh.max;
  uint32_t& s_t0 = sh.t0;
  uint32_t* s_wcnt = sh.wcnt;
  uint64_t* s_cand = sh.cand;
  uint32_t* s_hist = sh.hist;
  uint32_t* s_ctl = sh.ctl;
  uint32_t& s_nsel = sh.nsel;
  uint32_t* s_sel_key = sh.sel_key;
  int32_t* s_sel_blk = sh.sel_blk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t k = (uint32_t)kk;

  // Loads are unconditional (blocks past the row re-read its last block and
  // count as key 0), so all kPer of them are in flight together; a load
  // under a branch was waited for before the next one was issued.
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = min(tid + kSelThreads * i, nblk - 1);
    v[i] = srow[(int64_t)b * sc_s1];
  }
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    key[i] = tid + kSelThreads * i < nblk ? order_key(v[i]) : 0u;

  // Prefilter threshold T0: the k-th largest thread maximum.
  {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) m = max(m, key[i]);
    s_max[tid] = m;
  }
  __syncthreads();
  if (tid < 64) {
    uint32_t mm[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mm[j] = s_max[4 * lane + j];
    uint32_t t0 = 0u;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = t0 | (1u << bit);
      uint32_t cnt = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) cnt += (uint32_t)__popcll(__ballot(mm[j] >= c));
      if (cnt >= k) t0 = c;
    }
    if (lane == 0) s_t0 = t0;
  }
  __syncthreads();
  const uint32_t t0 = s_t0;
  const int wave = tid >> 6;
  {
    uint32_t cnt = 0u;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      cnt += (uint32_t)__popcll(__ballot(key[i] != 0u && key[i] >= t0));
    if (lane == 0) s_wcnt[wave] = cnt;
  }
  __syncthreads();
  uint32_t base = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    base += w < wave ? s_wcnt[w] : 0u;
    total += s_wcnt[w];
  }
  if (total <= (uint32_t)kSelCap) {
    // Compact the candidates (any order), then rank each against all.
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool c = key[i] != 0u && key[i] >= t0;
      const uint64_t bl = __ballot(c);
      if (c) {
        const uint32_t at = base + __builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(bl >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bl, 0u));
        s_cand[at] = pack_rank_key(key[i], tid + kSelThreads * i);
      }
      base += (uint32_t)__popcll(bl);
    }
    __syncthreads();
    for (int c = tid; c < (int)total; c += kSelThreads) {
      const uint64_t mine = s_cand[c];
      int rank = 0;
#pragma unroll 4
      for (int j = 0; j < (int)total; ++j) rank += s_cand[j] > mine ? 1 : 0;
      if (rank < kk) out[rank] = kMaxScoreBlocks - 1 - (int)(mine & (kMaxScoreBlocks - 1));
    }
    if (tid >= (int)total && tid < kk) out[tid] = -1;
    return;
  }

  uint32_t prefix = 0, mask = 0, need = k, ties = 0;
  bool take_all = false;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    s_hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (key[i] != 0u && (key[i] & mask) == prefix)
        atomicAdd(&s_hist[(key[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) pick_digit(s_hist, lane, need, s_ctl);
    __syncthreads();
    if (pass == 0 && s_ctl[3] <= k) {  // at most k selectable blocks: all of them
      take_all = true;
      break;
    }
    prefix |= s_ctl[0] << shift;
    mask |= 0xFFu << shift;
    need = s_ctl[1];
    ties = s_ctl[2];
    __syncthreads();
  }

  // Ties at the threshold key: keep the `need` lowest block ids (largest
  // inverted ids), found by radix select over the 14-bit inverted id.
  uint32_t inv_min = 0;
  if (!take_all && need < ties) {
    uint32_t ipref = 0, imask = 0;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 7 : 0;
      s_hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t inv = (uint32_t)(kMaxScoreBlocks - 1 - (tid + kSelThreads * i));
        if (key[i] == prefix && (inv & imask) == ipref)
          atomicAdd(&s_hist[(inv >> shift) & 127u], 1u);
      }
      __syncthreads();
      if (tid < 64) pick_digit(s_hist, lane, need, s_ctl);
      __syncthreads();
      ipref |= s_ctl[0] << shift;
      imask |= 127u << shift;
      need = s_ctl[1];
      __syncthreads();
    }
    inv_min = ipref;
  }

  if (tid == 0) s_nsel = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = tid + kSelThreads * i;
    const uint32_t inv = (uint32_t)(kMaxScoreBlocks - 1 - b);
    const bool take = take_all ? key[i] != 0u
                               : (key[i] > prefix || (key[i] == prefix && inv >= inv_min));
    if (take) {
      const uint32_t slot = atomicAdd(&s_nsel, 1u);
      if (slot < (uint32_t)kMaxTopk) {  // at most k <= kMaxTopk are taken
        s_sel_key[slot] = key[i];
        s_sel_blk[slot] = b;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int nsel = min((int)s_nsel, kk);
    if (lane < nsel) {
      const uint32_t mk = s_sel_key[lane];
      const int mb = s_sel_blk[lane];
      int rank = 0;
      for (int j = 0; j < nsel; ++j) {
        const uint32_t kj = s_sel_key[j];
        const int bj = s_sel_blk[j];
        rank += (kj > mk || (kj == mk && bj < mb)) ? 1 : 0;
      }
      out[rank] = mb;
    } else if (lane < kk) {
      out[lane] = -1;
    }
  }
}

}  // namespace msa
