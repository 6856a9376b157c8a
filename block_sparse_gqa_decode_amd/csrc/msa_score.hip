// Indexer block-max scorer and top-k block selector for gfx950.
//
// Scorer: score[h, b, t] = max over the group's q heads g and the keys i of
// block b visible at token t's position of q[t, h*G+g] . K[page(b), h, i],
// -inf for blocks that start after the position (TensorRT-LLM PR #17171
// "Custom decode kernels for MinimaxM3", indexer commit: per-block causal max
// of Q.K with a grid sized to the batch).  One wavefront owns one (request,
// kv head, block): it loads the block's K half once and evaluates every
// decode token of the request against it with the same S^T = K Q^T MFMA
// layout as the attend (16x16x32 bf16, q heads as the 16 columns).
//
// Selector: per (token, kv head), the k blocks with score > -inf in
// (score descending, block ascending) order, padded with -1 (same PR, strided
// selector; ties to the lower block index).  One wavefront per row runs k
// rounds; round i finds the best block strictly after winner i-1 in that
// order, so no per-element state is kept and any score stride works.
#include <climits>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kScoreWaves = 4;

template <bool kFp8>
struct BlockK;

template <>
struct BlockK<true> {
  u32x4_t k[8][2];  // [key tile][run of 16 fp8]
};

template <>
struct BlockK<false> {
  u32x4_t k[8][4];  // [key tile][chunk of 8 bf16]
};

template <bool kFp8>
__device__ __forceinline__ void k_operands(const BlockK<kFp8>& kb, int tile,
                                           bf16x8_t (&kf)[4]) {
  if constexpr (kFp8) {
    kf[0] = as_bf16x8(fp8x8_to_bf16x8(kb.k[tile][0].x, kb.k[tile][0].y));
    kf[1] = as_bf16x8(fp8x8_to_bf16x8(kb.k[tile][0].z, kb.k[tile][0].w));
    kf[2] = as_bf16x8(fp8x8_to_bf16x8(kb.k[tile][1].x, kb.k[tile][1].y));
    kf[3] = as_bf16x8(fp8x8_to_bf16x8(kb.k[tile][1].z, kb.k[tile][1].w));
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[c] = as_bf16x8(kb.k[tile][c]);
  }
}

template <bool kFp8>
__global__ __launch_bounds__(64 * kScoreWaves) void score_kernel(ScoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.x * kScoreWaves + wave;
  const int h = blockIdx.y;
  const int r = blockIdx.z;
  if (b >= p.max_blocks) return;
  float* sc = p.score + h * p.sc_s0 + (int64_t)b * p.sc_s1;

  if (r >= p.batch) {
    // Padding token rows: nothing is visible.
    for (int t = p.real_rows + lane; t < p.num_rows; t += 64) sc[t * p.sc_s2] = -INFINITY;
    return;
  }

  const int seq = p.seq_lens[r];
  const int t0 = r * p.dql;
  const int pos_last = seq - 1;
  bool vis = b < p.bt_stride && (int64_t)b * kPage <= pos_last;
  int pg = 0;
  if (vis) {
    pg = p.block_table[(int64_t)r * p.bt_stride + b];
    vis = pg >= 0 && pg < p.num_kv_blocks;
  }
  if (!vis) {
    for (int l = lane; l < p.dql; l += 64) sc[(int64_t)(t0 + l) * p.sc_s2] = -INFINITY;
    return;
  }
  const int nvis_max = min(kPage, pos_last - b * kPage + 1);
  const uint8_t* page_head = p.kv + pg * p.kv_s0 + h * p.kv_s1;

  BlockK<kFp8> kb;
#pragma unroll
  for (int tile = 0; tile < 8; ++tile) {
    const int kr = min(16 * tile + n, nvis_max - 1);
    const uint8_t* row = page_head + kr * p.kv_s2;
    if constexpr (kFp8) {
      kb.k[tile][0] = *reinterpret_cast<const u32x4_t*>(row + 16 * g);
      kb.k[tile][1] = *reinterpret_cast<const u32x4_t*>(row + 64 + 16 * g);
    } else {
      kb.k[tile][0] = *reinterpret_cast<const u32x4_t*>(row + 2 * (16 * g));
      kb.k[tile][1] = *reinterpret_cast<const u32x4_t*>(row + 2 * (16 * g + 8));
      kb.k[tile][2] = *reinterpret_cast<const u32x4_t*>(row + 2 * (64 + 16 * g));
      kb.k[tile][3] = *reinterpret_cast<const u32x4_t*>(row + 2 * (64 + 16 * g + 8));
    }
  }

  for (int l = 0; l < p.dql; ++l) {
    const int pos = seq - p.dql + l;
    const int nvis = min(kPage, pos - b * kPage + 1);
    float* dst = sc + (int64_t)(t0 + l) * p.sc_s2;
    if (nvis <= 0) {
      if (lane == 0) *dst = -INFINITY;
      continue;
    }
    bf16x8_t qf[4];
    if (n < p.group) {
      const uint16_t* qp =
          p.q + ((int64_t)(t0 + l) * p.hq + h * p.group + n) * kHeadDim;
      qf[0] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 16 * g));
      qf[1] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 16 * g + 8));
      qf[2] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g));
      qf[3] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(qp + 64 + 16 * g + 8));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) qf[c] = as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
    }
    float best = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      bf16x8_t kf[4];
      k_operands<kFp8>(kb, tile, kf);
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) s = mfma_bf16_16x16x32(kf[c], qf[c], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * tile + 4 * g + i;
        if (key < nvis && n < p.group) best = fmaxf(best, s[i] * p.k_scale);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
    if (lane == 0) *dst = best;
  }
}

__global__ __launch_bounds__(64) void select_kernel(SelectParams p) {
  const int lane = threadIdx.x;
  const int t = blockIdx.x / p.hkv;
  const int h = blockIdx.x - t * p.hkv;
  const float* s = p.score + h * p.sc_s0 + (int64_t)t * p.sc_s2;
  int32_t* out = p.topk_out + ((int64_t)t * p.hkv + h) * p.k;
  float pv = INFINITY;  // previous winner (score, block); nothing precedes it yet
  int pi = -1;
  for (int round = 0; round < p.k; ++round) {
    float bv = -INFINITY;
    int bi = INT_MAX;  // INT_MAX: no candidate
    for (int b = lane; b < p.max_blocks; b += 64) {
      const float v = s[(int64_t)b * p.sc_s1];
      if (!(v > -INFINITY)) continue;
      const bool after = v < pv || (v == pv && b > pi);
      if (!after) continue;
      if (v > bv || (v == bv && b < bi)) {
        bv = v;
        bi = b;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi == INT_MAX) {
      for (int rr = round + lane; rr < p.k; rr += 64) out[rr] = -1;
      break;
    }
    if (lane == 0) out[round] = bi;
    pv = bv;
    pi = bi;
  }
}

}  // namespace

hipError_t launch_score(const ScoreParams& p, bool fp8, hipStream_t stream) {
  const int pad = p.num_rows > p.real_rows ? 1 : 0;
  const dim3 grid((uint32_t)((p.max_blocks + kScoreWaves - 1) / kScoreWaves),
                  (uint32_t)p.hkv, (uint32_t)(p.batch + pad));
  if (fp8) {
    hipLaunchKernelGGL(score_kernel<true>, grid, dim3(64 * kScoreWaves), 0, stream, p);
  } else {
    hipLaunchKernelGGL(score_kernel<false>, grid, dim3(64 * kScoreWaves), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  const int64_t grid = (int64_t)p.num_rows * p.hkv;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3((uint32_t)grid), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
