// Launch parameters and launcher declarations shared by the C-ABI layer
// (msa_api.cpp) and the kernel translation units, and the unit -> XCD slot
// chunk size both the launchers and the kernels use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kPage = 128;      // tokens per KV page (= sparse block)
constexpr int kHeadDim = 128;   // head dimension
constexpr int kMaxGroup = 16;   // q heads per kv head handled by one MFMA tile
constexpr int kMaxTopk = 64;    // entries per top-k row
constexpr int kMaxSplits = 16;
constexpr int kMaxScoreBlocks = 16384;
constexpr int kMaxScoreBatch = 4096;   // requests per scorer launch (LDS prefix sum)
constexpr int kMaxScoreDql = 32;
constexpr int kMaxPrefills = 1 << 20;   // requests of one prefill plan
constexpr int kMaxTileRows = 4;        // token rows of a multi-row tile
constexpr int kMaxUnion = kMaxTileRows * kMaxTopk;   // pages of a tile's union
constexpr int kXcdSlots = 8;   // XCDs a launch is dealt across, round robin

// Single-row attend and merge: units are dealt to the XCD slots in chunks of
// consecutive units, so a request's neighbouring tokens and kv heads share
// one L2.  A chunk is up to 16 token rows' units (all kv heads) and at most
// an eighth of the launch, so work stays spread when requests differ in
// cost.  The launch then has ceil(units / (8 * chunk)) * chunk workgroups
// per slot and split; unit of (slot x, k-th workgroup) =
// ((k / chunk) * 8 + x) * chunk + k % chunk, each unit exactly once.
__host__ __device__ inline int xcd_chunk(int units, int hkv) {
  const int c = units / kXcdSlots < hkv * 16 ? units / kXcdSlots : hkv * 16;
  return c > 1 ? c : 1;
}

__host__ __device__ inline int xcd_unit(int units, int hkv, int slot, int k) {
  const int c = xcd_chunk(units, hkv);
  return ((k / c) * kXcdSlots + slot) * c + k % c;
}

inline int64_t xcd_groups(int64_t units, int hkv) {
  const int64_t c = xcd_chunk((int)units, hkv);
  return (units + kXcdSlots * c - 1) / (kXcdSlots * c) * c;
}

// Sparse row tiles: units (tile, kv head) are dealt to the XCD slots in
// chunks of kTileBlock consecutive tiles of one kv head, chunk c of the
// launch going to slot c % 8.  A request's tiles draw on the same pages per
// head, so a chunk's re-reads of a page meet in one L2 instead of two or more
// (the plain round robin spread a head's tiles over two XCDs).  Per split,
// the launch has tile_block_groups(tiles, hkv) workgroups per slot; the k-th
// on slot x takes tile_block_unit(tiles, hkv, x, k), -1 past the last tile.
constexpr int kTileBlock = 16;

__host__ __device__ inline int64_t tile_block_groups(int64_t tiles, int hkv) {
  const int64_t chunks = (tiles + kTileBlock - 1) / kTileBlock * hkv;
  return (chunks + kXcdSlots - 1) / kXcdSlots * kTileBlock;
}

__host__ __device__ inline int tile_block_unit(int tiles, int hkv, int slot, int k) {
  const int c = (k / kTileBlock) * kXcdSlots + slot;   // chunk of this workgroup
  const int block = c / hkv;
  const int h = c - block * hkv;
  const int tile = block * kTileBlock + k % kTileBlock;
  return tile < tiles ? tile * hkv + h : -1;
}

// Element formats (the values of msa_kv_dtype / msa_q_dtype).
constexpr int kKvBf16 = 0;
constexpr int kKvE4m3 = 1;     // OCP fp8 e4m3fn
constexpr int kKvE5m2 = 2;     // OCP fp8 e5m2
constexpr int kKvMxfp4 = 3;    // OCP MXFP4 head slots (e2m1 + E8M0 per 32 dims)
constexpr int kQBf16 = 0;
constexpr int kQE4m3 = 1;

struct AttendParams {
  const uint8_t* q;         // bf16 or fp8 e4m3fn [rows, hq, 128] (bytes)
  const uint8_t* kv;        // packed K|V base (bytes)
  // Strides in bytes: page, head, row.  For MXFP4 head slots: page, head
  // (to the head's K slot), and the K slot -> V slot offset.
  int64_t kv_s0, kv_s1, kv_s2;
  int64_t num_kv_blocks;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* topk;
  int64_t tk_s0, tk_s1, tk_s2;  // strides in elements
  uint16_t* out;            // bf16 [rows, hq, 128]
  float* part_o;            // fp32 [rows, hq, splits, 128]
  float* part_ml;           // fp32 [rows, hq, splits, 2] = (max, sum) in log2 units
  float scale_log2;         // sm_scale * q_scale * k_scale * log2(e)
  float v_scale;
  int32_t dql, real_rows, num_rows, hq, hkv, group, topk_k, splits, num_units;
  // Ragged prefill (null for decode): request r owns rows cu_q[r]..cu_q[r+1]-1,
  // its local token i sits at ctx_lens[r] + i; rows >= cu_q[num_reqs] are
  // padding.  real_rows is then num_rows and seq_lens / dql are unused.
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  int32_t num_reqs;
  // Multi-row tiles (tile kernel only): tile_dense selects every visible
  // block of request-aligned tiles instead of the rows' top-k union.
  int32_t tile_dense;
  // Sparse decode row tiles of at most 64 requests whose tiles never span two
  // requests: dispatch the requests' tiles longest request first (see
  // msa_tile.hip).
  int32_t len_order;
  // In-kernel split merge (single-row attend, 2..kMaxFusedSplits splits):
  // one arrival counter per unit, zero between launches; null = the merge
  // kernel combines the partials instead.
  int32_t* arrivals;
  // Single-row decode attend that selects its own top-k (null = read topk):
  // fp32 block scores [hkv, sel_max_blocks, rows] with element strides
  // sel_s0..2; the selection is also written to sel_topk_out
  // ([rows, hkv, topk_k], contiguous) when that is not null.
  const float* sel_score;
  int64_t sel_s0, sel_s1, sel_s2;
  int32_t sel_max_blocks;
  int32_t* sel_topk_out;
};

constexpr int kMaxFusedSplits = 4;

struct ScoreParams {
  const uint8_t* q;         // bf16 or fp8 e4m3fn [rows, hq, 128] (bytes)
  const uint8_t* kv;
  int64_t kv_s0, kv_s1, kv_s2;  // bytes, as in AttendParams
  int64_t num_kv_blocks;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  float* score;             // fp32 logical [hkv, max_blocks, rows]
  int64_t sc_s0, sc_s1, sc_s2;  // elements
  float qk_scale;           // q_scale * k_scale
  int32_t batch, dql, real_rows, num_rows, hq, hkv, group, max_blocks;
};

struct SelectParams {
  const float* score;
  int64_t sc_s0, sc_s1, sc_s2;
  int32_t* topk_out;        // int32 [rows, hkv, k]
  int32_t hkv, max_blocks, num_rows, k;
};

// kv_fmt: kKv*; q_fmt: kQ*.  An fp8 q needs an 8-bit or 4-bit KV format.
hipError_t launch_attend(const AttendParams& p, int kv_fmt, int q_fmt, hipStream_t stream);
hipError_t launch_merge(const AttendParams& p, hipStream_t stream);
// Multi-row tiles of tile_rows (2 or 4) token rows; p.num_units = tiles * hkv.
hipError_t launch_tile(const AttendParams& p, int kv_fmt, int q_fmt, int tile_rows,
                       hipStream_t stream);
// Row tiles of 8 token rows over 8-bit KV (e4m3 / e5m2), pages staged
// through an LDS ring; p.num_units = tiles * hkv.
hipError_t launch_union(const AttendParams& p, int kv_fmt, int q_fmt, int tile_rows,
                        hipStream_t stream);
hipError_t launch_score(const ScoreParams& p, int kv_fmt, int q_fmt, hipStream_t stream);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);
// fmt: kKvE4m3 or kKvE5m2
hipError_t launch_fp8_to_bf16(const uint8_t* in, uint16_t* out, int64_t n, int fmt,
                              hipStream_t stream);
// MXFP4 head-slot pages (strides in bytes: page, head, K -> V slot) -> bf16
// packed K|V rows [num_blocks, hkv, 128, 256], unscaled.
hipError_t launch_mxfp4_to_bf16(const uint8_t* kv, int64_t s0, int64_t s1, int64_t s2,
                                int64_t num_blocks, int hkv, uint16_t* out, hipStream_t stream);

}  // namespace msa
