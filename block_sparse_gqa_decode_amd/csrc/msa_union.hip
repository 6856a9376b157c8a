// Row-tile block-sparse attend for 8-bit KV caches on gfx950, with pages
// staged through an LDS ring by direct-to-LDS loads.
//
// What is computed is exactly the attend of msa_attend.hip: each token row
// attends, per kv head, the causally visible keys of its selected 128-token
// pages (vLLM API page "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparseImpl and the decode and prefill calls of
// MiniMaxM3SparseTritonImpl.forward; vLLM test file
// test_minimax_m3_msa_cutlass_sparse_decode.py, _make_topk), or every visible
// block in the dense variant (TensorRT-LLM PR #17171, dense-decode commit).
//
// Work decomposition.  A workgroup takes a tile of kR = 8 token rows for
// one kv head and walks the union of the rows' pages (each page once, with
// every row's visible count); dense tiles walk every block of their request.
// The tile's q rows (the GQA group of each token: kR x 16 MFMA rows in all)
// are staged in LDS.  Wavefront w owns keys [32w, 32w+32) of every page: it
// widens its 32 keys of K once per page for all rows, then for each row that
// sees the page runs S^T = K Q^T (16 keys x 16 q heads per MFMA tile), the
// mask and the online softmax, builds its V^T operands once and runs
// O^T += V^T P^T per row.  The kR rows' O live in the accumulators.
//
// Memory pipeline.  Each wavefront streams its own 32 rows of each page
// (32 x 256 bytes, the K and V halves of a packed fp8 row) into a private
// slice of a kD-stage LDS ring with 16-byte direct-to-LDS loads
// (global_load_lds_dwordx4: eight per page, 64 lanes x 16 bytes each, four
// full rows per instruction, so every request is a whole 256-byte row).  The
// loads of page i + kD - 1 are issued before page i is computed, so kD - 1
// pages per wavefront are in flight without holding any VGPRs; a wavefront
// waits (vmcnt) only for its own loads, so the page loop has no barrier.
// Rows past a page's visible count are not read: the load repeats the last
// visible row instead.
//
// LDS layout of a slice: row r (0..31) at 256 r; its sixteen 16-byte chunks
// are stored permuted, chunk c at position c ^ swz(r), where swz is a
// bijection of r mod 16 that keeps the K reads (16 rows, one chunk each) and
// the V reads (8-byte halves of 4 rows) free of bank conflicts.  The
// permutation is applied on the global side (each lane fetches the chunk
// that belongs at its LDS position), so the rows still load whole.
//
// Split-K over the page list writes the same fp32 partials as the other
// attend kernels, merged by the same merge kernel.
#include <type_traits>

#include "msa_device.h"
#include "msa_internal.h"
#include "msa_page.h"
#include "msa_rows.h"

namespace msa {
namespace {

constexpr uint32_t kRowBytes = 2 * kHeadDim;            // one packed fp8 K|V row
constexpr uint32_t kSliceBytes = kKeysPerWave * kRowBytes;  // a wavefront's rows
constexpr uint32_t kStageBytes = kWaves * kSliceBytes;  // one page

// Chunk permutation of slice row r: a bijection of r mod 16 that flips bit 3
// with bit 2, so the V reads of lane groups g and g^1 (rows 4g+j and 4g+4+j)
// land on complementary chunk halves.
__device__ __forceinline__ uint32_t swz(uint32_t r) {
  const uint32_t x = r & 15u;
  return x ^ (((x >> 2) & 1u) << 3);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(kN >= 0 && kN < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (kN & 15) | ((kN >> 4) << 14));
}

// A compiler barrier for memory operations: the direct-to-LDS loads write LDS
// behind the compiler's back, so LDS reads of a stage must not move above the
// wait for its loads, and the loads into a stage must not move above the
// reads of its previous page.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// One 16-byte direct-to-LDS load per lane: lane L's 16 bytes at base + voff
// land at LDS byte lds_addr + 16 L.  Written as inline assembly so that the
// compiler does not track it: it would otherwise wait for every load into LDS
// before any LDS read, draining the ring (its alias information does not reach
// these loads).  The explicit vmcnt waits of the ring are what orders a stage's
// reads after its loads; the memory clobber keeps the compiler from moving LDS
// accesses across the load.  No output register: the data goes to LDS only.
// Wait states: 5 after a VALU write of the base SGPRs (v_readfirstlane), 1
// between the M0 write and the load that reads it.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds_addr) {
  // Both scalar operands are wave-uniform; readfirstlane puts them in SGPRs
  // (the constraint alone would not when the compiler cannot prove it).
  lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
  const uint64_t b = (uint64_t)(size_t)base;
  const uint32_t b_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t b_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  base = (const uint8_t*)(size_t)(((uint64_t)b_hi << 32) | b_lo);
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// The eight direct-to-LDS loads of one wavefront's 32 rows of a page.
// `page` is the page-head base (wave-uniform), `lim` the last visible row of
// the page, `kbase` the wavefront's first row, `slice` its LDS slice.
__device__ __forceinline__ void stage_rows(const uint8_t* page, uint32_t row_stride, int lim,
                                           int kbase, int lane, uint8_t* slice) {
  const uint32_t lds = lds_offset(slice);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lr = 4u * i + (uint32_t)(lane >> 4);      // slice row of this lane
    const uint32_t c = (uint32_t)(lane & 15);                // its LDS chunk
    const uint32_t row = (uint32_t)min(kbase + (int)lr, lim);
    const uint32_t off = __umul24(row, row_stride) + 16u * (c ^ swz(lr));
    dma16(page, off, lds + 1024u * i);
  }
}

// The PageRegs<1> registers of the register-ring kernels, read from a slice:
// K runs (head dims 16g.., 64+16g..) of rows 16 tau + n and V head dims
// 8n..8n+7 of the eight key slots.
__device__ __forceinline__ void read_slice(const uint8_t* slice, int n, int g,
                                           PageRegs<1>& r) {
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const uint32_t lr = 16u * tau + n;
    const uint8_t* row = slice + lr * kRowBytes;
    const uint32_t s = swz(lr);
    r.k[tau][0] = *reinterpret_cast<const u32x4_t*>(row + 16u * ((uint32_t)g ^ s));
    r.k[tau][1] = *reinterpret_cast<const u32x4_t*>(row + 16u * ((4u + g) ^ s));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lr = (uint32_t)key_of_slot(g, j);
    const uint32_t chunk = (8u + ((uint32_t)n >> 1)) ^ swz(lr);
    r.v[j] = *reinterpret_cast<const u32x2_t*>(slice + lr * kRowBytes + 16u * chunk +
                                               8u * (n & 1));
  }
}

// The token row of tile position w (-1 when the position holds no row), as
// in the register-ring tile kernel: dense tiles are request-aligned.
__device__ __forceinline__ int union_row(const AttendParams& p, int tile, int w, int kR) {
  if (p.tile_dense) {
    const int tpr = (p.dql + kR - 1) / kR;
    const int req_tiles = (p.real_rows / p.dql) * tpr;
    if (tile >= req_tiles) {
      const int t = p.real_rows + (tile - req_tiles) * kR + w;
      return t < p.num_rows ? t : -1;
    }
    const int r = tile / tpr;
    const int local = (tile - r * tpr) * kR + w;
    return local < p.dql ? r * p.dql + local : -1;
  }
  return tile * kR + w;
}

// Page list entry: physical page (0 when no row sees it) and one byte per
// tile row with that row's visible count (0 = the row does not see it).
struct ListEntry {
  int32_t page;
  uint32_t nv_lo;   // rows 0..3
  uint32_t nv_hi;   // rows 4..7
  int32_t pad;
};

template <int kR>
constexpr int kStages = kR == 8 ? 3 : 4;

// A wavefront's online-softmax state for the tile's rows.
template <int kR>
struct RowState {
  float m_run[kR];
  float l_part[kR];
  f32x4_t o[kR][8];
};

// Row w's visible count of a page from its list entry's row bytes.
__device__ __forceinline__ int row_nv(uint32_t nlo, uint32_t nhi, int w) {
  return (int)(((w < 4 ? nlo : nhi) >> (8 * (w & 3))) & 0xffu);
}

template <int kJ>
__device__ __forceinline__ uint8_t* pick_stage(uint8_t* __restrict__ s0, uint8_t* __restrict__ s1,
                                               uint8_t* __restrict__ s2, uint8_t* __restrict__ s3) {
  if constexpr (kJ == 0) return s0;
  else if constexpr (kJ == 1) return s1;
  else if constexpr (kJ == 2) return s2;
  else return s3;
}

// One page for the wavefront: its 32 keys from the slice, K widened once,
// then S^T, mask and online softmax for each row that sees the page, V^T
// once and P V for those rows.
template <int kKv, int kQ, int kR>
__device__ __forceinline__ void compute_page(const uint8_t* __restrict__ slice,
                                             const uint8_t* __restrict__ q_lds, uint32_t nlo,
                                             uint32_t nhi, int kbase, int n, int g,
                                             float scale_log2, RowState<kR>& rs) {
  constexpr int kQBytes = kHeadDim * (kQ == kQE4m3 ? 1 : 2);
  constexpr int kQStride = kQBytes + 16;
  const uint32_t ksh = 8u * g;
  PageRegs<1> pr;
  read_slice(slice, n, g, pr);
  bf16x8_t pb[kR];
  {
    bf16x8_t kf[2][4];
    if constexpr (kQ != kQE4m3) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) widen_k_tile<kKv>(pr, tau, ksh, kf[tau]);
    }
#pragma unroll
    for (int w = 0; w < kR; ++w) {
      const int nv = row_nv(nlo, nhi, w);
      if (nv > kbase) {
        QRegs<kQ> qw;
        load_q_operand<1, kQ>(qw, q_lds + (w * 16 + n) * kQStride, true, g);
        f32x4_t s[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          if constexpr (kQ == kQE4m3) {
            s[tau] = score_tile_fp8q<kKv>(pr, qw, tau, ksh);
          } else {
            s[tau] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) s[tau] = mfma_bf16_16x16x32(kf[tau][c], qw.f[c], s[tau]);
          }
        }
        float z[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
          for (int e = 0; e < 4; ++e) z[4 * tau + e] = s[tau][e];
        }
        if (kbase + kKeysPerWave > nv) {
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kbase + 16 * tau + 4 * g + e >= nv) z[4 * tau + e] = -INFINITY;
          }
        }
        pb[w] = softmax_step(z, scale_log2, rs.m_run[w], rs.l_part[w], rs.o[w]);
      }
    }
  }
  u32x4_t vt[8];
  build_vt<kKv>(pr, 0u, vt);
#pragma unroll
  for (int w = 0; w < kR; ++w) {
    if (row_nv(nlo, nhi, w) > kbase) {
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8)
        rs.o[w][t8] = mfma_bf16_16x16x32(as_bf16x8(vt[t8]), pb[w], rs.o[w][t8]);
    }
  }
}

// The page ring over list entries [u0, u1) (LDS list indexes).  Every LDS
// object the walk touches comes in as its own restrict pointer, so each
// access carries alias-scope information and the compiler can tell a
// stage's reads apart from the loads still in flight into the other stages
// (without it, it waits for every load to LDS before any LDS read).  The
// stage of each step is a template index for the same reason: a stage
// chosen at run time would be "based on" every stage pointer.
template <int kKv, int kQ, int kR>
__device__ __forceinline__ void ring_walk(uint8_t* __restrict__ st0, uint8_t* __restrict__ st1,
                                          uint8_t* __restrict__ st2, uint8_t* __restrict__ st3,
                                          const uint8_t* __restrict__ q_lds,
                                          const ListEntry* __restrict__ list, int u0, int u1,
                                          const uint8_t* head_base, int64_t page_stride,
                                          uint32_t row_stride, int kbase, int lane,
                                          float scale_log2, RowState<kR>& rs) {
  constexpr int kD = kStages<kR>;
  const int n = lane & 15;
  const int g = lane >> 4;
  const uint32_t my_off = (uint32_t)(kbase / kKeysPerWave) * kSliceBytes;
  uint32_t blo[kD], bhi[kD];
  // Issues the loads of list entry u into stage kS; keeps its row counts.
  auto fetch = [&](auto S, int u) {
    constexpr int kS = decltype(S)::value;
    const ListEntry e = list[u];
    const int pg = __builtin_amdgcn_readfirstlane(e.page);
    const uint32_t nlo = (uint32_t)__builtin_amdgcn_readfirstlane((int)e.nv_lo);
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)e.nv_hi);
    blo[kS] = nlo;
    bhi[kS] = nhi;
    uint32_t vmax = 0;
#pragma unroll
    for (int w = 0; w < kR; ++w) vmax = max(vmax, (uint32_t)row_nv(nlo, nhi, w));
    lds_order();
    stage_rows(head_base + (int64_t)pg * page_stride, row_stride, (int)max(vmax, 1u) - 1, kbase,
               lane, pick_stage<kS>(st0, st1, st2, st3) + my_off);
  };
  // Step kJ of the unrolled ring: prefetch into the stage the previous page
  // left, wait for this page's loads, compute it.
  auto step = [&](auto J, int cur) {
    constexpr int kJ = decltype(J)::value;
    fetch(std::integral_constant<int, (kJ + kD - 1) % kD>{}, min(cur + kD - 1, u1 - 1));
    wait_vmcnt<8 * (kD - 1)>();
    lds_order();
    const uint32_t nlo = blo[kJ], nhi = bhi[kJ];
    bool any = false;
#pragma unroll
    for (int w = 0; w < kR; ++w) any |= row_nv(nlo, nhi, w) > kbase;
    if (any)
      compute_page<kKv, kQ, kR>(pick_stage<kJ>(st0, st1, st2, st3) + my_off, q_lds, nlo, nhi,
                                kbase, n, g, scale_log2, rs);
  };
  if (u0 < u1) {
    fetch(std::integral_constant<int, 0>{}, u0);
    fetch(std::integral_constant<int, 1>{}, min(u0 + 1, u1 - 1));
    if constexpr (kD > 3) fetch(std::integral_constant<int, 2>{}, min(u0 + 2, u1 - 1));
    for (int i = u0;; i += kD) {
      step(std::integral_constant<int, 0>{}, i);
      if (i + 1 >= u1) break;
      step(std::integral_constant<int, 1>{}, i + 1);
      if (i + 2 >= u1) break;
      step(std::integral_constant<int, 2>{}, i + 2);
      if (i + 3 >= u1) break;
      if constexpr (kD > 3) {
        step(std::integral_constant<int, 3>{}, i + 3);
        if (i + 4 >= u1) break;
      }
    }
  }
  // Every load into the ring has landed before the ring is refilled or
  // reused for the merge buffers.
  wait_vmcnt<0>();
  lds_order();
}

template <int kKv, int kQ, int kR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
union_kernel(AttendParams p) {
  constexpr int kD = kStages<kR>;
  constexpr int kMaxEnt = kR * kMaxTopk;       // a tile's (row, slot) entries
  constexpr int kQBytes = kHeadDim * (kQ == kQE4m3 ? 1 : 2);
  constexpr int kQStride = kQBytes + 16;       // padded: 16 heads' reads spread over banks
  // The ring, one array per stage (distinct objects, so the compiler can tell
  // a stage's reads from the loads in flight into the others); after the
  // page loop the first stages hold the wavefronts' merge buffers.
  __shared__ __align__(1024) uint8_t s_st0[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st1[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st2[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st3[kD > 3 ? kStageBytes : 16];

  __shared__ __align__(16) ListEntry s_list[kMaxEnt];
  __shared__ __align__(16) int32_t s_ent_page[kMaxEnt];
  __shared__ __align__(16) int32_t s_ent_nv[kMaxEnt];
  __shared__ __align__(16) uint8_t s_q[kR][16][kQStride];
  __shared__ int32_t s_row_r[kR], s_row_pos[kR];
  __shared__ int32_t s_wave_cnt[kWaves];
  __shared__ int32_t s_nlist;
  // Merge buffers: wavefronts 0 and 1 put their O in stage 0, 2 and 3 in
  // stage 1; the maxima and sums go to stage 2.
  typedef float OBuf[16][kHeadDim + kOPad];
  static_assert(2 * sizeof(OBuf) <= kStageBytes, "two wavefronts' O fit in a stage");
  static_assert(sizeof(float) * kWaves * 16 * 2 <= kStageBytes, "merge sums fit in a stage");
  auto s_o = [&](int w) -> OBuf& {
    return reinterpret_cast<OBuf*>(w < 2 ? s_st0 : s_st1)[w & 1];
  };
  float(*s_m)[16] = reinterpret_cast<float(*)[16]>(s_st2);
  float(*s_l)[16] = s_m + kWaves;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (tile, kv head, split), splits of a (tile, head) on one XCD.
  const int xslot = blockIdx.x % kXcdSlots;
  const int q8 = blockIdx.x / kXcdSlots;
  const int split = q8 % p.splits;
  const int unit = (q8 / p.splits) * kXcdSlots + xslot;
  if (unit >= p.num_units) return;
  const int tile = unit / p.hkv;
  const int h = unit - tile * p.hkv;
  const int head0 = h * p.group;

  if (tid < kR) {
    const int t = union_row(p, tile, tid, kR);
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
  // Stage q (zeros for dead rows and q heads >= G); the barriers of the list
  // build below order these writes before the first read.
  constexpr int kQChunks = kQBytes / 16;
  for (int c = tid; c < kR * 16 * kQChunks; c += kThreads) {
    const int w = c / (16 * kQChunks);
    const int rem = c - w * (16 * kQChunks);
    const int qh = rem / kQChunks;
    const int off = (rem - qh * kQChunks) * 16;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (s_row_r[w] >= 0 && qh < p.group) {
      const int64_t q_row = (int64_t)union_row(p, tile, w, kR) * p.hq + head0 + qh;
      v = *reinterpret_cast<const u32x4_t*>(p.q + q_row * kQBytes + off);
    }
    *reinterpret_cast<u32x4_t*>(&s_q[w][qh][off]) = v;
  }

  int npages;
  int dense_r = -1;
  if (!p.tile_dense) {
    // Union of the rows' selections.  Entry e = w * k + j is (row w, slot j):
    // its physical page (-1 for an empty, invalid or padding slot) and the
    // row's visible count of it.
    const int k = p.topk_k;
    const int kq = (k + 3) & ~3;  // slots scanned per row (the pad is -1)
    const int ne = kR * kMaxTopk;
    for (int e = tid; e < ne; e += kThreads) {
      const int w = e / kMaxTopk;
      const int j = e - w * kMaxTopk;
      const int r = s_row_r[w];
      const int pos = s_row_pos[w];
      int page = -1, nv = 0;
      if (r >= 0 && j < k) {
        const int t = union_row(p, tile, w, kR);
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
    // Each entry scans every entry: it opens a list slot if it is the first
    // naming its page, with every row's largest visible count of the page.
    // Slots follow entry order (prefix counts over the threads' passes).
    int base = 0;
    for (int e0 = 0; e0 < ne; e0 += kThreads) {
      const int e = e0 + tid;
      bool first = false;
      uint32_t lo = 0, hi = 0;
      int page = -1;
      if (e < ne) page = s_ent_page[e];
      if (page >= 0) {
        int first_e = e;
#pragma unroll
        for (int w = 0; w < kR; ++w) {
          int v = 0;
          for (int j = 0; j < kq; j += 4) {
            const int e2 = w * kMaxTopk + j;
            const int4 pg4 = *reinterpret_cast<const int4*>(&s_ent_page[e2]);
            const int4 nv4 = *reinterpret_cast<const int4*>(&s_ent_nv[e2]);
            if (pg4.x == page) { first_e = min(first_e, e2); v = max(v, nv4.x); }
            if (pg4.y == page) { first_e = min(first_e, e2 + 1); v = max(v, nv4.y); }
            if (pg4.z == page) { first_e = min(first_e, e2 + 2); v = max(v, nv4.z); }
            if (pg4.w == page) { first_e = min(first_e, e2 + 3); v = max(v, nv4.w); }
          }
          if (w < 4) lo |= (uint32_t)v << (8 * w);
          else hi |= (uint32_t)v << (8 * (w - 4));
        }
        first = first_e == e;
      }
      const uint64_t bal = __ballot(first);
      if (lane == 0) s_wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int before = base;
      for (int w2 = 0; w2 < wave; ++w2) before += s_wave_cnt[w2];
      if (first) {
        const int slot = before + __popcll(bal & ((1ull << lane) - 1ull));
        s_list[slot] = ListEntry{page, lo, hi, 0};
      }
      for (int w2 = 0; w2 < kWaves; ++w2) base += s_wave_cnt[w2];
      __syncthreads();
    }
    npages = base;
  } else {
    dense_r = s_row_r[0];
    int pos_max = -1;
#pragma unroll
    for (int w = 0; w < kR; ++w) pos_max = max(pos_max, s_row_pos[w]);
    npages = dense_r >= 0 && pos_max >= 0 ? min(pos_max / kPage + 1, p.bt_stride) : 0;
  }

  // This split's share of the page list.
  const int lo = (int)((int64_t)npages * split / p.splits);
  const int hi = (int)((int64_t)npages * (split + 1) / p.splits);

  RowState<kR> rs;
#pragma unroll
  for (int w = 0; w < kR; ++w) {
    rs.m_run[w] = -INFINITY;
    rs.l_part[w] = 0.f;
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) rs.o[w][t8] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int kbase = wave * kKeysPerWave;
  const uint8_t* head_base = p.kv + h * p.kv_s1;
  const uint32_t row_stride = (uint32_t)p.kv_s2;
  const int32_t* dense_row = p.block_table + (int64_t)(dense_r >= 0 ? dense_r : 0) * p.bt_stride;

  // Dense tiles stage their list in chunks of kMaxEnt table entries; a
  // sparse list is one chunk, already staged.
  for (int c0 = lo; c0 < hi; c0 += kMaxEnt) {
    const int c1 = min(hi, c0 + kMaxEnt);
    if (p.tile_dense) {
      __syncthreads();  // the previous chunk's entries are no longer read
      for (int u = c0 + tid; u < c1; u += kThreads) {
        const int raw = dense_row[u];
        const bool ok = raw >= 0 && raw < p.num_kv_blocks;
        uint32_t nlo = 0, nhi = 0;
#pragma unroll
        for (int w = 0; w < kR; ++w) {
          int v = 0;
          if (ok && s_row_pos[w] >= 0) v = max(0, min(kPage, s_row_pos[w] - u * kPage + 1));
          if (w < 4) nlo |= (uint32_t)v << (8 * w);
          else nhi |= (uint32_t)v << (8 * (w - 4));
        }
        s_list[u - c0] = ListEntry{(nlo | nhi) != 0 ? raw : 0, nlo, nhi, 0};
      }
      __syncthreads();
    }
    const int lbase = p.tile_dense ? c0 : 0;  // list index of LDS entry 0
    ring_walk<kKv, kQ, kR>(s_st0, s_st1, s_st2, s_st3, &s_q[0][0][0], s_list, c0 - lbase,
                           c1 - lbase, head_base, p.kv_s0, row_stride, kbase, lane,
                           p.scale_log2, rs);
  }
  __syncthreads();  // all wavefronts are done with the ring

  // Row by row: merge the four wavefronts' states, then write the bf16 row
  // (one split), the fp32 partial (several), or zeros for a padding row.
  const int qr = tid >> 4;
  const int d0 = (tid & 15) * 8;
#pragma unroll
  for (int w = 0; w < kR; ++w) {
    const int t = union_row(p, tile, w, kR);
    const bool live = s_row_r[w] >= 0;
    const float l_run = wave_sum_xor_16_32(rs.l_part[w]);
    if (w > 0) __syncthreads();  // the previous row's merge buffers are no longer read
    if (g == 0) {
      s_m[wave][n] = rs.m_run[w];
      s_l[wave][n] = l_run;
    }
#pragma unroll
    for (int t8 = 0; t8 < 8; ++t8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_o(wave)[n][32 * g + 8 * e + t8] = rs.o[w][t8][e];
    }
    __syncthreads();
    if (t < 0 || t >= p.num_rows || qr >= p.group) continue;
    const int64_t row = (int64_t)t * p.hq + head0 + qr;
    if (!live) {
      if (split == 0)
        *reinterpret_cast<u32x4_t*>(p.out + row * kHeadDim + d0) = u32x4_t{0u, 0u, 0u, 0u};
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
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // An empty wavefront weighs 0 (multiplied in, so a NaN sum propagates).
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      const float ew = mw[w2] == -INFINITY ? 0.f : fast_exp2(mw[w2] - M);
      L += ew * s_l[w2][qr];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ew * s_o(w2)[qr][d0 + e];
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
hipError_t launch_union_fmt(const AttendParams& p, int tile_rows, dim3 gd, hipStream_t stream) {
  if (tile_rows != 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((union_kernel<kKv, kQ, 8>), gd, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_union(const AttendParams& p, int kv_fmt, int q_fmt, int tile_rows,
                        hipStream_t stream) {
  const int64_t groups = ((int64_t)p.num_units + kXcdSlots - 1) / kXcdSlots;
  const int64_t grid = groups * kXcdSlots * p.splits;
  if (grid <= 0) return hipSuccess;
  const dim3 gd((uint32_t)grid);
  if (q_fmt == kQE4m3) {
    if (kv_fmt == kKvE4m3) return launch_union_fmt<kKvE4m3, kQE4m3>(p, tile_rows, gd, stream);
    if (kv_fmt == kKvE5m2) return launch_union_fmt<kKvE5m2, kQE4m3>(p, tile_rows, gd, stream);
    return hipErrorInvalidValue;
  }
  if (kv_fmt == kKvE4m3) return launch_union_fmt<kKvE4m3, kQBf16>(p, tile_rows, gd, stream);
  if (kv_fmt == kKvE5m2) return launch_union_fmt<kKvE5m2, kQBf16>(p, tile_rows, gd, stream);
  return hipErrorInvalidValue;
}

}  // namespace msa
