// Block-sparse GQA decode attend for gfx950.
//
// What is computed: each decode token attends, per kv head, only the keys of
// its indexer-selected 128-token pages that are causally visible at its
// position (vLLM API page "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparseImpl; vLLM test file test_minimax_m3_msa_cutlass_sparse_decode.py,
// _make_topk), with split-K over the selected blocks, fp32 partials and zeroed
// padding rows (TensorRT-LLM PR #17171, flash-decoding commit).
//
// Decode and prefill share the kernel: a decode token row t belongs to
// request t / dql at position seq_len - dql + t % dql (vLLM test file
// test_minimax_m3_msa_cutlass_sparse_decode.py, _make_topk); a ragged prefill
// row belongs to the request r with cu_seqlens_q[r] <= t < cu_seqlens_q[r+1]
// (found by a wave-uniform binary search) at position context_lens[r] +
// t - cu_seqlens_q[r] (vLLM API page
// "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparsePrefillMetadata and the prefill call of
// MiniMaxM3SparseTritonImpl.forward).
//
// Work decomposition.  A unit is one (token row t, kv head h); its G q heads
// are the 16 rows of one MFMA tile.  A workgroup of 4 wavefronts handles one
// unit's share (split) of its live pages; wavefront w owns keys
// [32w, 32w+32) of every page, so the workgroup reads each page once and the
// four wavefronts keep separate online-softmax states that are merged through
// LDS at the end.
//
// Register layouts (16x16x32 bf16 MFMA, lane l, n = l % 16, g = l / 16):
//  * S^T = K Q^T: A = K rows (key n of a 16-key tile), B = Q^T (q row n).  The
//    contraction slot (g, c, j) of chunk c maps to head dim
//    d = 64*(c/2) + 16*g + 8*(c%2) + j, so a lane reads two contiguous 16-dim
//    runs of its key row.  The accumulator gives lane l the scores of keys
//    4g..4g+3 of the tile for q row n.
//  * O^T += V^T P^T: B = P^T comes straight from the two S^T accumulators of
//    the wavefront's 32 keys (contraction slot j of group g = key
//    4g+j for j<4, 16+4g+(j-4) for j>=4).  A = V^T uses the same key slots;
//    its row m of d-tile t8 is head dim 8m+t8, so lane l loads the 8
//    contiguous head dims 8n..8n+7 of each of its 8 keys and a byte permute
//    transposes them into the 8 d-tiles.  The accumulator then holds
//    O[q row n][32g + 8i + t8] for i < 4, t8 < 8: 32 contiguous outputs.
//
// Split-K: with S > 1 splits every workgroup produces an fp32 partial
// (unnormalised O, running max and sum in log2 units) in the plan's arena.
// With 2..4 splits the last split of a unit to finish merges them in this
// kernel (fused_merge: system-scope stores and loads of the partials, a
// system-scope arrival counter; a device-scope fence would write back the
// whole L2 on this part); with more, a second small kernel merges them by
// log-sum-exp.  Workgroup ids are laid out so each XCD slot takes chunks of
// consecutive units with all their splits (the dispatcher deals consecutive
// workgroups to the 8 XCDs in turn), so a request's tokens and heads, which
// share pages, meet in one L2.
//
// Pipeline: each wavefront keeps two pages in registers, one in flight while
// it computes the other, as a ring unrolled twice so every buffer index is
// static and each wait covers only the page computed.  (Deeper rings, eight
// wavefronts per workgroup over alternate pages, or two workgroups per unit
// over half the q heads each measured no faster: with one workgroup per CU
// the step is bound by HBM latency and bandwidth, not by issue.)
//
// Formats: K|V entries are bf16, OCP fp8 e4m3fn, OCP fp8 e5m2 or MXFP4; q is bf16 or
// fp8 e4m3fn with a per-tensor q scale (vLLM API page
// "vllm.models.minimax_m3.nvidia.msa_cutlass_sparse_decode":
// msa_cutlass_sparse_decode(query_fp8, ..., q_scale_float, ...)).  With a bf16
// q the 8-bit K is widened to bf16 in registers and S^T uses the bf16 MFMA
// above.  With an fp8 q, S^T of a 16-key tile is one 16x16x128 fp8 MFMA on the
// K bytes as loaded: both operands take head dims 16g..16g+15 then
// 64+16g..64+16g+15 in lane group g, the same runs the K loads already fetch.
// The q, k and softmax scales fold into one log2-domain factor.  P V stays a
// bf16 MFMA (V widened to bf16).
//
// 4-bit pages (an MXFP4 analogue of the NVFP4 head-slot page of the vLLM test
// file, _make_nvfp4_kv_cache): head h's K slot holds 128 rows of 64 bytes of
// e2m1 codes, then 128 rows of four E8M0 scales, one per 32 head dims; its V
// slot follows at a fixed offset.  A K lane takes the 32 contiguous head dims
// 32g..32g+31 of its key row, which is one MX block: with an fp8 q they are
// the A operand of the scaled 16x16x128 MFMA (fp4 A, fp8 B) with the block's
// scale code as the lane's A scale; with a bf16 q they widen to bf16 with that
// scale, and q takes the same 32-dim chunks.  A V lane widens the 8 dims
// 8n..8n+7 of each of its keys with the key's block scale, then the byte
// permute transposes them as for 8-bit V.
//
// NaN safety: rows past a page's visible count are never loaded (row index
// clamped to the last visible row) and their scores are set to -inf, so stale
// cache bytes cannot reach the MFMAs.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_page.h"
#include "msa_rows.h"
#include "msa_select.h"

namespace msa {
namespace {

// Reads through this pointer type go to the scalar cache when the index is
// wave-uniform.
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Log-sum-exp merge of the split partials of one (token row, q head) and the
// bf16 store of head dims d0..d0+7.
__device__ __forceinline__ void merge_splits(const AttendParams& p, int64_t row, int d0) {
  const float* ml = p.part_ml + row * p.splits * 2;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // A split that saw no key weighs 0 (its sum and O are 0); the weight is
  // multiplied in rather than the split skipped, so a NaN sum still reaches L.
  {
    for (int s = 0; s < p.splits; ++s) {
      const float ms = ml[2 * s];
      const float e = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      L += e * ml[2 * s + 1];
      const float* po = p.part_o + (row * p.splits + s) * kHeadDim + d0;
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(po);
      const f32x4_t b = *reinterpret_cast<const f32x4_t*>(po + 4);
      acc[0] += e * a.x; acc[1] += e * a.y; acc[2] += e * a.z; acc[3] += e * a.w;
      acc[4] += e * b.x; acc[5] += e * b.y; acc[6] += e * b.z; acc[7] += e * b.w;
    }
  }
  store_row(p.out + row * kHeadDim + d0, acc, L, p.v_scale);
}

// In-kernel split merge.  Every split writes its partial with system-scope
// stores (sc0 sc1: written through to memory, acknowledged there), waits for
// them, and bumps the unit's arrival counter with a system-scope atomic; the
// split that arrives last reads every partial back with system-scope loads
// (sc0 sc1: no cache keeps a stale copy), combines them in split order with
// the merge kernel's arithmetic, writes the bf16 row and resets the counter.
// No workgroup waits for another and no cache is written back or invalidated
// (a device-scope release fence writes back the whole L2 on this part).
constexpr int kSysCoherent = 0x11;        // buffer cache policy: sc0 | sc1
constexpr int kWaitVmem = 0x0F70;         // s_waitcnt vmcnt(0)

template <int kS>
__device__ __forceinline__ void combine_splits(__amdgpu_buffer_rsrc_t ro,
                                               __amdgpu_buffer_rsrc_t rm, int qr, int d0,
                                               uint16_t* dst, float v_scale) {
  f32x2_t m_l[kS];
  f32x4_t a[kS], b[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const int slot = qr * kS + s;
    m_l[s] = __builtin_bit_cast(
        f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, slot * 8, 0, kSysCoherent));
    a[s] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                           ro, (slot * kHeadDim + d0) * 4, 0, kSysCoherent));
    b[s] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                           ro, (slot * kHeadDim + d0 + 4) * 4, 0, kSysCoherent));
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kS; ++s) M = fmaxf(M, m_l[s].x);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // Unconditional (an empty split weighs 0, see merge_fixed), so the O and
  // (m, l) read-backs go out together: one memory round trip, not two.
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const float e = m_l[s].x == -INFINITY ? 0.f : fast_exp2(m_l[s].x - M);
    L += e * m_l[s].y;
    acc[0] += e * a[s].x; acc[1] += e * a[s].y; acc[2] += e * a[s].z; acc[3] += e * a[s].w;
    acc[4] += e * b[s].x; acc[5] += e * b[s].y; acc[6] += e * b[s].z; acc[7] += e * b[s].w;
  }
  store_row(dst, acc, L, v_scale);
}

// The fused epilogue of one split workgroup of `unit`, whose q rows are
// urow0 .. urow0 + rows - 1; thread (qr, d0) owns head dims d0..d0+7 of row
// qr when `owner`.  s_last is a workgroup-shared flag.
__device__ __forceinline__ void fused_merge(const AttendParams& p, int unit, int64_t urow0,
                                            int rows, int split, bool owner, int qr, int d0,
                                            const float (&acc)[8], float M, float L,
                                            int& s_last) {
  const int S = p.splits;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      p.part_o + urow0 * S * kHeadDim, (short)0, rows * S * kHeadDim * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + urow0 * S * 2, (short)0, rows * S * 2 * 4, kRsrcWord3);
  if (owner) {
    const int slot = qr * S + split;
    const f32x4_t lo = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
    const f32x4_t hi = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, lo), ro,
                                           (slot * kHeadDim + d0) * 4, 0, kSysCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, hi), ro,
                                           (slot * kHeadDim + d0 + 4) * 4, 0, kSysCoherent);
    if (d0 == 0)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, f32x2_t{M, L}), rm,
                                            slot * 8, 0, kSysCoherent);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(p.arrivals + unit, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_SYSTEM) == S - 1;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0)
    __hip_atomic_store(p.arrivals + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (!owner) return;
  uint16_t* dst = p.out + (urow0 + qr) * kHeadDim + d0;
  if (S == 2) combine_splits<2>(ro, rm, qr, d0, dst, p.v_scale);
  else if (S == 3) combine_splits<3>(ro, rm, qr, d0, dst, p.v_scale);
  else combine_splits<4>(ro, rm, qr, d0, dst, p.v_scale);
}

// kSelPer > 0 (decode rows): the workgroup selects its row's top-k from the
// block scores itself (select_row, kSelPer scores per thread) instead of
// reading a top-k row, so an indexed step needs no separate selector launch
// and no top-k round trip through memory.
template <int kKv, int kQ, bool kVarlen, int kSelPer = 0>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendParams p) {
  constexpr int kKind = kv_kind(kKv);
  static_assert(kSelPer == 0 || (kThreads == kSelThreads && !kVarlen), "selecting attend");
  __shared__ SelShared s_selsh;
  __shared__ int32_t s_sel[kMaxTopk];
  __shared__ int32_t s_page[kMaxTopk];
  __shared__ int32_t s_nvis[kMaxTopk];
  __shared__ int32_t s_nlive;
  __shared__ int s_last;
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][kHeadDim + kOPad];
  // The selecting attend's staged block-table row (see below).
  constexpr bool kStageTable = kSelPer > 0;
  constexpr int kTableCap = kStageTable ? kTableLoads * kThreads : 1;
  __shared__ int32_t s_table[kTableCap];
  __shared__ int32_t s_len;

  // Every kernel argument the prologue reads, fetched as one batch of scalar
  // loads: left to itself the compiler loads them in three dependent
  // batches, each a scalar-cache miss at the start of the launch.
  asm volatile("" ::"s"(p.q), "s"(p.kv), "s"(p.kv_s0), "s"(p.kv_s1), "s"(p.kv_s2),
               "s"(p.num_kv_blocks), "s"(p.block_table), "s"(p.seq_lens), "s"(p.topk));
  asm volatile("" ::"s"(p.tk_s0), "s"(p.tk_s1), "s"(p.tk_s2), "s"(p.bt_stride), "s"(p.dql),
               "s"(p.real_rows), "s"(p.hq), "s"(p.hkv), "s"(p.group), "s"(p.topk_k),
               "s"(p.splits), "s"(p.num_units));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  // Workgroups are dealt to the 8 XCDs in turn; each XCD slot takes chunks of
  // consecutive units (xcd_chunk) with all splits of a unit.  Neighbouring
  // units are a request's tokens and heads, which share pages and the
  // block-table row, so they meet in one XCD's L2.
  const int xslot = blockIdx.x % kXcdSlots;
  const int q8 = blockIdx.x / kXcdSlots;
  const int split = q8 % p.splits;
  const int unit = xcd_unit(p.num_units, p.hkv, xslot, q8 / p.splits);
  if (unit >= p.num_units) return;
  const int t = unit / p.hkv;
  const int h = unit - t * p.hkv;
  const int rows = p.group;  // q heads of the unit = MFMA rows in use
  const int head0 = h * p.group;

  // Decode rows are computed inline (the request index stays a scalar; the
  // position is read with the top-k row below); prefill rows use the binary
  // search.
  int r = 0, pos = 0;
  bool live;
  if constexpr (!kVarlen) {
    live = t < p.real_rows;
    r = live ? t / p.dql : 0;
  } else {
    live = locate_token<1>(p, t, r, pos);
  }
  if (!live) {
    // Padding row: exact zeros, written once.
    if (split == 0) {
      const int qr = tid >> 4;
      const int d0 = (tid & 15) * 8;
      if (qr < p.group) {
        uint16_t* dst = p.out + ((int64_t)t * p.hq + h * p.group + qr) * kHeadDim + d0;
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{0u, 0u, 0u, 0u};
      }
      // A padding row selects nothing (as the selector gives for its -inf
      // scores).
      if (kSelPer > 0 && p.sel_topk_out != nullptr && tid < p.topk_k)
        p.sel_topk_out[((int64_t)t * p.hkv + h) * p.topk_k + tid] = -1;
    }
    return;
  }

  // Resolve the top-k row into the ordered list of live pages.  The lane's
  // top-k entry (a vector load at a clamped lane: a single-row plan always
  // has a top-k row) and a decode row's length (a scalar load through the
  // constant address space) are both in flight before either is used, and
  // the filter takes no short cuts, so neither read waits behind the other:
  // top-k and length, then the block table, then the pages.
  //
  // The selecting attend instead reads its row's block-table entries (the
  // first kTableCap, coalesced across the workgroup) and length together
  // with the score row it selects from, so the selected pages follow from
  // LDS: 32.2 -> 31.9 us a launch on the indexed full step.  The top-k
  // attend gained nothing from the same staging (its table read is not what
  // bounds the launch), so it keeps the chain.
  const int li = lane < p.topk_k ? lane : 0;
  int b_raw = 0;
  int table_n = 0;
  if constexpr (kStageTable) {
    table_n = min(p.bt_stride, kTableCap);
    // Clamped, unconditional loads (entries past the row's end are never
    // stored): a per-lane condition would branch around every load.
    int32_t tv[kTableLoads];
    const int32_t* trow = p.block_table + (int64_t)r * p.bt_stride;
#pragma unroll
    for (int i = 0; i < kTableLoads; ++i) tv[i] = trow[min(tid + i * kThreads, table_n - 1)];
    // The length travels with the table entries (every thread stores the
    // same value), so its read cannot be sunk behind them.
    const int len = p.seq_lens[r];
    select_row<kSelPer>(p.sel_score + h * p.sel_s0 + (int64_t)t * p.sel_s2, p.sel_s1,
                        p.sel_max_blocks, p.topk_k, s_selsh, s_sel);
#pragma unroll
    for (int i = 0; i < kTableLoads; ++i) {
      const int e = tid + i * kThreads;
      if (e < table_n) s_table[e] = tv[i];
    }
    s_len = len;
    __syncthreads();
    pos = s_len - p.dql + (t - r * p.dql);
    if (p.sel_topk_out != nullptr && split == 0 && tid < p.topk_k)
      p.sel_topk_out[((int64_t)t * p.hkv + h) * p.topk_k + tid] = s_sel[tid];
    b_raw = s_sel[li];
  }
  if (wave == 0) {
    bool live = false;
    int page = 0, nvis = 0;
    if constexpr (!kStageTable) {
      b_raw = p.topk[t * p.tk_s0 + h * p.tk_s1 + li * p.tk_s2];
      if constexpr (!kVarlen)
        pos = ((const const_i32*)p.seq_lens)[r] - p.dql + (t - r * p.dql);
    }
    const int b = lane < p.topk_k ? b_raw : -1;
    if ((b >= 0) & (b < p.bt_stride) & ((int64_t)b * kPage <= pos)) {
      int pg;
      if constexpr (kStageTable) {
        // An LDS read for every lane, a global read only for blocks past
        // the staged entries (kept apart, so no flat load picks between
        // them).
        pg = s_table[min(b, table_n - 1)];
        if (b >= table_n) {
          pg = p.block_table[(int64_t)r * p.bt_stride + b];
          asm volatile("" : "+v"(pg));
        }
      } else {
        pg = p.block_table[(int64_t)r * p.bt_stride + b];
      }
      if (pg >= 0 && pg < p.num_kv_blocks) {
        live = true;
        page = pg;
        nvis = min(kPage, pos - b * kPage + 1);
      }
    }
    const uint64_t mask = __ballot(live);
    if (live) {
      const int idx = __popcll(mask & ((1ull << lane) - 1ull));
      s_page[idx] = page;
      s_nvis[idx] = nvis;
    }
    if (lane == 0) s_nlive = __popcll(mask);
  }

  // Q^T operand of q row n (see load_q_operand for the head-dim slots).
  QRegs<kQ> qf;
  const int64_t q_row = (int64_t)t * p.hq + head0 + n;
  load_q_operand<kKind, kQ>(qf, p.q + q_row * kHeadDim * (kQ == kQE4m3 ? 1 : 2), n < rows,
                            g);
  __syncthreads();

  const int nlive = s_nlive;
  const int per = (nlive + p.splits - 1) / p.splits;
  const int lo = min(nlive, split * per);
  const int hi = min(nlive, lo + per);
  const int kbase = wave * kKeysPerWave;
  const uint8_t* head_base = p.kv + h * p.kv_s1;
  const uint32_t row_stride = (uint32_t)p.kv_s2;
  LaneRows lr = lane_rows<kKind>(kbase, n, g);
  lane_offsets(lr, row_stride);

  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) o[t8] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // kDepth-deep ring over the live pages (see the header comment).  Loads are
  // issued unconditionally: a page past the split's end re-reads the split's
  // last page (an L2 hit) and an inactive wavefront's rows all clamp to one
  // visible row, so no load sits on a conditional path before a wait.  Page
  // ids and visible counts are wave-uniform and live in scalar registers.
  if (lo < hi) {
    // A page's visible count is read with its page id when its loads are
    // issued and kept in a scalar register until the page is used.
    PageRegs<kKind> buf[kDepth];
    int bnv[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth - 1; ++j) {
      const int pi = min(lo + j, hi - 1);
      const int pg = __builtin_amdgcn_readfirstlane(s_page[pi]);
      bnv[j] = __builtin_amdgcn_readfirstlane(s_nvis[pi]);
      load_page_rows<kKind>(buf[j], head_base + (int64_t)pg * p.kv_s0, row_stride, bnv[j], lr);
    }
    for (int i = lo;; i += kDepth) {
#pragma unroll
      for (int j = 0; j < kDepth; ++j) {
        const int cur = i + j;
        if (cur >= hi) goto pages_done;
        const int pn = min(cur + kDepth - 1, hi - 1);
        const int nx = (j + kDepth - 1) % kDepth;
        const int pg = __builtin_amdgcn_readfirstlane(s_page[pn]);
        bnv[nx] = __builtin_amdgcn_readfirstlane(s_nvis[pn]);
        load_page_rows<kKind>(buf[nx], head_base + (int64_t)pg * p.kv_s0, row_stride, bnv[nx],
                              lr);
        const int nv = bnv[j];
        if (kbase < nv)
          attend_page<kKv, kQ>(buf[j], qf, lr, kbase, nv, g, p.scale_log2, m_run, l_part, o);
      }
    }
  }
pages_done:

  // Merge the wavefronts' states through LDS.
  const float l_run = wave_sum_xor_16_32(l_part);
  if (g == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_run;
  }
#pragma unroll
  for (int t8 = 0; t8 < 8; ++t8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][n][32 * g + 8 * i + t8] = o[t8][i];
  }
  __syncthreads();

  const int qr = tid >> 4;
  const int d0 = (tid & 15) * 8;
  const bool owner = qr < rows;
  float M = -INFINITY;
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  if (owner) {
    float mw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = s_m[w][qr];
      M = fmaxf(M, mw[w]);
    }
    // A wavefront that saw no key weighs 0 (multiplied in, not skipped, so a
    // NaN sum from NaN cache entries propagates as the definition gives).
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - M);
      L += e * s_l[w][qr];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += e * s_o[w][qr][d0 + k];
    }
  }

  const int64_t row = (int64_t)t * p.hq + head0 + qr;
  if (p.splits == 1) {
    if (owner) store_row(p.out + row * kHeadDim + d0, acc, L, p.v_scale);
    return;
  }
  if (p.arrivals != nullptr) {
    fused_merge(p, unit, (int64_t)t * p.hq + head0, rows, split, owner, qr, d0, acc, M, L,
                s_last);
    return;
  }

  if (owner) {
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

// Merge pass: one workgroup per (token row, kv head) unit, placed on the XCD
// slot that holds the unit in the single-row attend (xcd_unit) so the
// partials come from the L2 they were written through;
// thread (q row, 8 head dims).  All of a row's partial loads are issued
// before any is used.
template <int kS>
__device__ __forceinline__ void merge_fixed(const AttendParams& p, int64_t row, int d0) {
  const float* ml = p.part_ml + row * kS * 2;
  const float* po = p.part_o + row * kS * kHeadDim + d0;
  f32x2_t m_l[kS];
  f32x4_t a[kS], b[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    m_l[s] = *reinterpret_cast<const f32x2_t*>(ml + 2 * s);
    a[s] = *reinterpret_cast<const f32x4_t*>(po + s * kHeadDim);
    b[s] = *reinterpret_cast<const f32x4_t*>(po + s * kHeadDim + 4);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kS; ++s) M = fmaxf(M, m_l[s].x);
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  // Unconditional, so every partial load is issued before the first use: a
  // split with no key has max -inf, sum 0 and zero O, so weight 0, and a row
  // whose splits all saw nothing sums to L = 0 (stored as zeros).
#pragma unroll
  for (int s = 0; s < kS; ++s) {
    const float e = m_l[s].x == -INFINITY ? 0.f : fast_exp2(m_l[s].x - M);
    L += e * m_l[s].y;
    acc[0] += e * a[s].x; acc[1] += e * a[s].y; acc[2] += e * a[s].z; acc[3] += e * a[s].w;
    acc[4] += e * b[s].x; acc[5] += e * b[s].y; acc[6] += e * b[s].z; acc[7] += e * b[s].w;
  }
  store_row(p.out + row * kHeadDim + d0, acc, L, p.v_scale);
}

// At most two wavefronts per SIMD asked of the compiler, so a 16-split row keeps
// all its partial loads in flight (150 VGPRs) instead of batching them.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void merge_kernel(AttendParams p) {
  const int units = p.num_rows * p.hkv;
  const int unit = xcd_unit(units, p.hkv, (int)(blockIdx.x % kXcdSlots),
                            (int)(blockIdx.x / kXcdSlots));
  if (unit >= units) return;
  const int t = unit / p.hkv;
  const int h = unit - t * p.hkv;
  const int qr = threadIdx.x >> 4;
  // Padding rows were written as zeros by the attend.  A row is real when it
  // lies below the real rows (decode) or below the last chunk boundary
  // (prefill); no position is needed here.
  const bool real = p.cu_q != nullptr ? t < p.cu_q[p.num_reqs] : t < p.real_rows;
  if (!real || qr >= p.group) return;
  const int64_t row = (int64_t)t * p.hq + h * p.group + qr;
  const int d0 = (threadIdx.x & 15) * 8;
  switch (p.splits) {
    case 2: merge_fixed<2>(p, row, d0); break;
    case 3: merge_fixed<3>(p, row, d0); break;
    case 4: merge_fixed<4>(p, row, d0); break;
    case 8: merge_fixed<8>(p, row, d0); break;
    case 16: merge_fixed<16>(p, row, d0); break;
    default: merge_splits(p, row, d0); break;
  }
}

// 8-bit codes -> bf16 through the same conversion helper the attend uses.
template <int kFmt>
__global__ __launch_bounds__(256) void fp8_to_bf16_kernel(const uint8_t* in, uint16_t* out,
                                                          int64_t n) {
  const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (base >= n) return;
  uint32_t w = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (base + b < n) w |= (uint32_t)in[base + b] << (8 * b);
  const u32x4_t v = f8x8_to_bf16x8<kFmt>(w, 0u);
  const uint16_t vals[4] = {(uint16_t)(v.x & 0xffffu), (uint16_t)(v.x >> 16),
                            (uint16_t)(v.y & 0xffffu), (uint16_t)(v.y >> 16)};
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (base + b < n) out[base + b] = vals[b];
}

// MXFP4 head-slot pages -> packed bf16 K|V rows [num_blocks, hkv, 128, 256]
// (block scales applied, global scales not).  Item = (page, head, row, side,
// 32-dim block): 16 data bytes and one scale in, 64 bytes out.
__global__ __launch_bounds__(256) void mxfp4_to_bf16_kernel(const uint8_t* kv, int64_t s0,
                                                            int64_t s1, int64_t s2,
                                                            int64_t num_blocks, int hkv,
                                                            uint16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= num_blocks * hkv * kPage * 8) return;
  const int blk = (int)(i & 3);
  const int side = (int)((i >> 2) & 1);
  const int64_t rowid = i >> 3;                     // (page * hkv + head) * 128 + row
  const int row = (int)(rowid % kPage);
  const int64_t ph = rowid / kPage;
  const int h = (int)(ph % hkv);
  const int64_t page = ph / hkv;
  const uint8_t* slot = kv + page * s0 + h * s1 + side * s2;
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(slot + row * kF4RowBytes + 16 * blk);
  const float sc = e8m0_to_f32(slot[kF4ScaleBase + row * 4 + blk]);
  uint16_t* dst = out + rowid * (2 * kHeadDim) + side * kHeadDim + 32 * blk;
  *reinterpret_cast<u32x4_t*>(dst) = f4x8_to_bf16x8(d.x, sc);
  *reinterpret_cast<u32x4_t*>(dst + 8) = f4x8_to_bf16x8(d.y, sc);
  *reinterpret_cast<u32x4_t*>(dst + 16) = f4x8_to_bf16x8(d.z, sc);
  *reinterpret_cast<u32x4_t*>(dst + 24) = f4x8_to_bf16x8(d.w, sc);
}

}  // namespace

template <bool kVarlen>
static hipError_t launch_attend_rows(const AttendParams& p, int kv_fmt, int q_fmt, dim3 gd,
                                     hipStream_t stream) {
  const dim3 bd(kThreads);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3)
      hipLaunchKernelGGL((attend_kernel<kKvE4m3, kQE4m3, kVarlen>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvE5m2)
      hipLaunchKernelGGL((attend_kernel<kKvE5m2, kQE4m3, kVarlen>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvMxfp4)
      hipLaunchKernelGGL((attend_kernel<kKvMxfp4, kQE4m3, kVarlen>), gd, bd, 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else {
    if (kv_fmt == kKvE4m3)
      hipLaunchKernelGGL((attend_kernel<kKvE4m3, kQBf16, kVarlen>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvE5m2)
      hipLaunchKernelGGL((attend_kernel<kKvE5m2, kQBf16, kVarlen>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvMxfp4)
      hipLaunchKernelGGL((attend_kernel<kKvMxfp4, kQBf16, kVarlen>), gd, bd, 0, stream, p);
    else
      hipLaunchKernelGGL((attend_kernel<kKvBf16, kQBf16, kVarlen>), gd, bd, 0, stream, p);
  }
  return hipGetLastError();
}

template <int kSelPer>
static hipError_t launch_attend_select(const AttendParams& p, int kv_fmt, int q_fmt, dim3 gd,
                                       hipStream_t stream) {
  const dim3 bd(kThreads);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3)
      hipLaunchKernelGGL((attend_kernel<kKvE4m3, kQE4m3, false, kSelPer>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvE5m2)
      hipLaunchKernelGGL((attend_kernel<kKvE5m2, kQE4m3, false, kSelPer>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvMxfp4)
      hipLaunchKernelGGL((attend_kernel<kKvMxfp4, kQE4m3, false, kSelPer>), gd, bd, 0, stream,
                         p);
    else
      return hipErrorInvalidValue;
  } else {
    if (kv_fmt == kKvE4m3)
      hipLaunchKernelGGL((attend_kernel<kKvE4m3, kQBf16, false, kSelPer>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvE5m2)
      hipLaunchKernelGGL((attend_kernel<kKvE5m2, kQBf16, false, kSelPer>), gd, bd, 0, stream, p);
    else if (kv_fmt == kKvMxfp4)
      hipLaunchKernelGGL((attend_kernel<kKvMxfp4, kQBf16, false, kSelPer>), gd, bd, 0, stream,
                         p);
    else
      hipLaunchKernelGGL((attend_kernel<kKvBf16, kQBf16, false, kSelPer>), gd, bd, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendParams& p, int kv_fmt, int q_fmt, hipStream_t stream) {
  const int64_t grid = xcd_groups(p.num_units, p.hkv) * kXcdSlots * p.splits;
  if (grid <= 0) return hipSuccess;
  const dim3 gd((uint32_t)grid);
  if (p.sel_score != nullptr) {
    // 8 scores per thread cover 2048 blocks (a 256k-token context); 64 the
    // largest score row.
    if (p.cu_q != nullptr) return hipErrorInvalidValue;
    return p.sel_max_blocks <= 8 * kSelThreads
               ? launch_attend_select<8>(p, kv_fmt, q_fmt, gd, stream)
               : launch_attend_select<64>(p, kv_fmt, q_fmt, gd, stream);
  }
  return p.cu_q != nullptr ? launch_attend_rows<true>(p, kv_fmt, q_fmt, gd, stream)
                           : launch_attend_rows<false>(p, kv_fmt, q_fmt, gd, stream);
}

hipError_t launch_merge(const AttendParams& p, hipStream_t stream) {
  // Units (token row, kv head), padding rows included (they return at once),
  // dealt to XCD slots in chunks as in the single-row attend.
  const int64_t units = (int64_t)p.num_rows * p.hkv;
  if (units <= 0) return hipSuccess;
  const int64_t grid = xcd_groups(units, p.hkv) * kXcdSlots;
  hipLaunchKernelGGL(merge_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_mxfp4_to_bf16(const uint8_t* kv, int64_t s0, int64_t s1, int64_t s2,
                                int64_t num_blocks, int hkv, uint16_t* out, hipStream_t stream) {
  const int64_t items = num_blocks * hkv * kPage * 8;
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 255) / 256;
  hipLaunchKernelGGL(mxfp4_to_bf16_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, kv, s0,
                     s1, s2, num_blocks, hkv, out);
  return hipGetLastError();
}

hipError_t launch_fp8_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, int fmt,
                              hipStream_t stream) {
  const int64_t grid = (n + 1023) / 1024;
  if (fmt == kKvE5m2)
    hipLaunchKernelGGL((fp8_to_bf16_kernel<kKvE5m2>), dim3((uint32_t)grid), dim3(256), 0,
                       stream, in, out, n);
  else
    hipLaunchKernelGGL((fp8_to_bf16_kernel<kKvE4m3>), dim3((uint32_t)grid), dim3(256), 0,
                       stream, in, out, n);
  return hipGetLastError();
}

}  // namespace msa
