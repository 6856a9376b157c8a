// C ABI of the block-sparse GQA decode library (declared in
// include/msa_sparse_decode.h).  Argument checks are plain host code and run
// before any HIP call, so misuse is reported the same way with or without a
// GPU.  The plan mirrors the plan cache of the vLLM API page
// "vllm.models.minimax_m3.nvidia.msa_cutlass_sparse_decode"
// (MSACutlassDecodePlanCache: one plan per static shape whose device state
// keeps stable addresses across CUDA/HIP graph replays); its only device state
// is the fp32 split-K partial arena (TensorRT-LLM PR #17171, flash-decoding
// commit: partials from a persistent buffer arena).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "msa_internal.h"
#include "msa_plan.h"
#include "msa_sparse_decode.h"

namespace msa {
// Defined in msa_probe.hip.
hipError_t launch_read_runs(const uint8_t* base, int64_t buffer_bytes, const int64_t* run_off,
                            const int32_t* run_len, const int32_t* wg_first, int32_t num_runs,
                            int32_t num_workgroups, uint32_t* out, hipStream_t stream);
}  // namespace msa

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace msa {

msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

}  // namespace msa

using msa::fail;
using msa::ok;

namespace {

msa_status device_fail(hipError_t e, const char* what) {
  return fail(MSA_ERR_DEVICE, "%s failed: %s", what, hipGetErrorString(e));
}

// Bytes per kv_strides unit: bf16 elements, fp8 codes, or (MXFP4) bytes.
int64_t elem_bytes(int32_t kv_dtype) { return kv_dtype == MSA_KV_BF16 ? 2 : 1; }

// One MXFP4 head slot: 128 rows x 64 code bytes + 128 rows x 4 scale bytes.
constexpr int64_t kMxfp4SlotBytes = msa::kPage * (msa::kHeadDim / 2 + msa::kHeadDim / 32);

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Scale arguments: finite, and q/k scales positive (the kernels take maxima
// of raw dot products before applying them).
msa_status check_scales(float q_scale, float k_scale) {
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale))
    return fail(MSA_ERR_INVALID_ARG, "scales must be finite");
  if (!(q_scale > 0.f) || !(k_scale > 0.f))
    return fail(MSA_ERR_INVALID_ARG, "q_scale and k_scale must be positive");
  return MSA_OK;
}

msa_status check_kv(const void* kv_cache, const int64_t kv_strides[4], int64_t num_kv_blocks,
                    int32_t kv_dtype) {
  if (kv_cache == nullptr) return fail(MSA_ERR_INVALID_ARG, "kv_cache is NULL");
  if (kv_strides == nullptr) return fail(MSA_ERR_INVALID_ARG, "kv_strides is NULL");
  if (num_kv_blocks < 1) return fail(MSA_ERR_INVALID_ARG, "num_kv_blocks must be >= 1");
  if (num_kv_blocks > INT32_MAX) return fail(MSA_ERR_UNSUPPORTED, "num_kv_blocks exceeds 2^31-1");
  if (kv_strides[3] != 1)
    return fail(MSA_ERR_INVALID_ARG, "kv_cache last-dim stride must be 1 (got %lld)",
                (long long)kv_strides[3]);
  if (!aligned16(kv_cache)) return fail(MSA_ERR_INVALID_ARG, "kv_cache is not 16-byte aligned");
  if (kv_dtype == MSA_KV_MXFP4) {
    for (int d = 0; d < 3; ++d) {
      if (kv_strides[d] < 1 || kv_strides[d] % 16 != 0)
        return fail(MSA_ERR_INVALID_ARG, "MXFP4 kv_cache stride %d (%lld bytes) must be a "
                    "positive multiple of 16", d, (long long)kv_strides[d]);
    }
    if (kv_strides[2] < kMxfp4SlotBytes)
      return fail(MSA_ERR_INVALID_ARG, "MXFP4 K -> V slot offset %lld is shorter than a slot "
                  "(8704 bytes)", (long long)kv_strides[2]);
    if (kv_strides[2] > (1 << 24))
      return fail(MSA_ERR_UNSUPPORTED, "MXFP4 K -> V slot offset above 16 MiB");
    return MSA_OK;
  }
  const int64_t eb = elem_bytes(kv_dtype);
  for (int d = 0; d < 3; ++d) {
    if (kv_strides[d] < 1)
      return fail(MSA_ERR_INVALID_ARG, "kv_cache stride %d must be positive", d);
    if ((kv_strides[d] * eb) % 16 != 0)
      return fail(MSA_ERR_INVALID_ARG, "kv_cache stride %d (%lld elements) is not a multiple "
                  "of 16 bytes", d, (long long)kv_strides[d]);
  }
  // The kernels form row offsets with 24-bit multiplies.
  if (kv_strides[2] * eb >= (1 << 24))
    return fail(MSA_ERR_UNSUPPORTED, "kv_cache row stride must be below 16 MiB");
  if (kv_strides[2] < 2 * msa::kHeadDim)
    return fail(MSA_ERR_INVALID_ARG, "kv_cache row stride %lld is shorter than a packed K|V "
                "row (256 elements)", (long long)kv_strides[2]);
  return MSA_OK;
}

// Split-K only when there are too few work units to give every CU a
// workgroup: each split costs a partial write plus a merge launch, which pays
// off only below one unit per CU.  Dense page lists are long (every visible
// block), so they split further.
int32_t choose_splits(const msa_decode_shape* s, int64_t units, bool dense) {
  if (s->num_splits > 0) return s->num_splits;
  const int64_t target = dense ? 1024 : 256;
  const int32_t cap = dense ? msa::kMaxSplits : (s->topk_blocks < 8 ? s->topk_blocks : 8);
  int32_t splits = 1;
  while (units * splits < target && splits * 2 <= cap) splits *= 2;
  return splits;
}

}  // namespace

namespace msa {

// Checks shared by the plan and the indexer entry point.
msa_status check_common_shape(const msa_decode_shape* s) {
  if (s == nullptr) return fail(MSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 1) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", s->batch);
  if (s->decode_query_len < 1 || s->decode_query_len > 32)
    return fail(MSA_ERR_INVALID_ARG, "decode_query_len must be in 1..32 (got %d)",
                s->decode_query_len);
  const int64_t real = (int64_t)s->batch * s->decode_query_len;
  if (real > (1 << 24))
    return fail(MSA_ERR_UNSUPPORTED, "batch*decode_query_len = %lld exceeds 2^24",
                (long long)real);
  if (s->num_token_rows != 0 && s->num_token_rows < real)
    return fail(MSA_ERR_INVALID_ARG,
                "num_token_rows (%d) must be 0 or >= batch*decode_query_len (%lld)",
                s->num_token_rows, (long long)real);
  if (s->num_token_rows > (1 << 24))
    return fail(MSA_ERR_UNSUPPORTED, "num_token_rows exceeds 2^24");
  if (s->page_table_stride < 1)
    return fail(MSA_ERR_INVALID_ARG, "page_table_stride must be >= 1 (got %d)",
                s->page_table_stride);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(MSA_ERR_INVALID_ARG, "head counts must be >= 1 (got %d q, %d kv)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads / s->num_kv_heads > msa::kMaxGroup)
    return fail(MSA_ERR_UNSUPPORTED, "GQA group %d exceeds %d q heads per kv head",
                s->num_q_heads / s->num_kv_heads, msa::kMaxGroup);
  if (s->num_q_heads > 1024)
    return fail(MSA_ERR_UNSUPPORTED, "num_q_heads exceeds 1024");
  if (s->page_size != msa::kPage)
    return fail(MSA_ERR_UNSUPPORTED, "page_size must be 128 (got %d)", s->page_size);
  if (s->head_dim != msa::kHeadDim)
    return fail(MSA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", s->head_dim);
  if (s->kv_dtype != MSA_KV_BF16 && s->kv_dtype != MSA_KV_FP8_E4M3 &&
      s->kv_dtype != MSA_KV_FP8_E5M2 && s->kv_dtype != MSA_KV_MXFP4)
    return fail(MSA_ERR_INVALID_ARG, "unknown kv_dtype %d", s->kv_dtype);
  if (s->q_dtype != MSA_Q_BF16 && s->q_dtype != MSA_Q_FP8_E4M3)
    return fail(MSA_ERR_INVALID_ARG, "unknown q_dtype %d", s->q_dtype);
  if (s->q_dtype == MSA_Q_FP8_E4M3 && s->kv_dtype == MSA_KV_BF16)
    return fail(MSA_ERR_UNSUPPORTED, "an fp8 q needs an fp8 (e4m3 or e5m2) or MXFP4 KV cache");
  return MSA_OK;
}

}  // namespace msa

using msa::check_common_shape;
using msa::DeviceGuard;

extern "C" {

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_last_error(void) { return g_last_error.c_str(); }

static msa_status make_plan(const msa_decode_shape* shape, bool prefill, int32_t real_rows,
                            int device, msa_plan* plan_out);

msa_status msa_sparse_decode_plan(const msa_decode_shape* shape, int device, msa_plan* plan_out) {
  if (plan_out == nullptr) return fail(MSA_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  msa_status st = check_common_shape(shape);
  if (st != MSA_OK) return st;
  return make_plan(shape, false, shape->batch * shape->decode_query_len, device, plan_out);
}

// The kernel a plan uses: rows per workgroup (1 = the single-row attend) and
// the number of workgroups per split.
static msa_status choose_tiles(const msa_decode_shape* s, bool prefill, bool dense,
                               int32_t num_rows, int32_t* tile_rows, int64_t* units) {
  int32_t tr = s->tile_rows;
  if (tr != 0 && tr != 1 && tr != 2 && tr != 4 && tr != 8)
    return fail(MSA_ERR_INVALID_ARG, "tile_rows must be 0 (auto), 1, 2, 4 or 8 (got %d)", tr);
  const bool kv8 = s->kv_dtype == MSA_KV_FP8_E4M3 || s->kv_dtype == MSA_KV_FP8_E5M2;
  if (tr == 8 && !kv8)
    return fail(MSA_ERR_UNSUPPORTED, "8-row tiles need an 8-bit (fp8 e4m3 or e5m2) KV cache");
  if (tr == 0) {
    // Measured on one MI355X: rows that share many pages (long decode query
    // lengths, prefill chunks) gain from 2-row tiles; dense decode, where every
    // row of a request shares every page, from 4-row tiles; rows that share
    // few pages run faster one per workgroup.
    if (dense) tr = s->decode_query_len <= 2 ? 2 : 4;
    else tr = (prefill || s->decode_query_len >= 8) ? 2 : 1;
  }
  if (dense && tr == 1)
    return fail(MSA_ERR_UNSUPPORTED, "dense decode runs on multi-row tiles (tile_rows 2 or 4)");
  int64_t tiles;
  if (tr == 1) tiles = num_rows;
  else if (dense)  // request-aligned tiles, then tiles of padding rows
    tiles = (int64_t)s->batch * ((s->decode_query_len + tr - 1) / tr) +
            ((int64_t)num_rows - (int64_t)s->batch * s->decode_query_len + tr - 1) / tr;
  else tiles = ((int64_t)num_rows + tr - 1) / tr;
  *tile_rows = tr;
  *units = tiles * s->num_kv_heads;
  return MSA_OK;
}

msa_status msa_sparse_prefill_plan(const msa_prefill_shape* pshape, int device,
                                   msa_plan* plan_out) {
  if (plan_out == nullptr) return fail(MSA_ERR_INVALID_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  if (pshape == nullptr) return fail(MSA_ERR_INVALID_ARG, "shape is NULL");
  if (pshape->num_prefills < 1)
    return fail(MSA_ERR_INVALID_ARG, "num_prefills must be >= 1 (got %d)", pshape->num_prefills);
  if (pshape->num_prefills > msa::kMaxPrefills)
    return fail(MSA_ERR_UNSUPPORTED, "num_prefills exceeds %d", msa::kMaxPrefills);
  if (pshape->num_token_rows < 1)
    return fail(MSA_ERR_INVALID_ARG, "num_token_rows must be >= 1 (got %d)",
                pshape->num_token_rows);
  // The shared shape checks, with a placeholder query length: every row is
  // potentially real until cu_seqlens_q says otherwise on the device.
  msa_decode_shape s{};
  s.batch = pshape->num_prefills;
  s.decode_query_len = 1;
  s.num_token_rows = pshape->num_token_rows;
  s.page_table_stride = pshape->page_table_stride;
  s.num_q_heads = pshape->num_q_heads;
  s.num_kv_heads = pshape->num_kv_heads;
  s.page_size = pshape->page_size;
  s.head_dim = pshape->head_dim;
  s.topk_blocks = pshape->topk_blocks;
  s.kv_dtype = pshape->kv_dtype;
  s.num_splits = pshape->num_splits;
  s.q_dtype = pshape->q_dtype;
  s.tile_rows = pshape->tile_rows;
  if (s.num_token_rows > (1 << 24)) return fail(MSA_ERR_UNSUPPORTED, "num_token_rows exceeds 2^24");
  const int32_t keep_rows = s.num_token_rows;
  s.num_token_rows = 0;  // batch*1 may exceed the rows; checked above instead
  msa_status st = check_common_shape(&s);
  if (st != MSA_OK) return st;
  s.num_token_rows = keep_rows;
  s.decode_query_len = 0;
  return make_plan(&s, true, keep_rows, device, plan_out);
}

}  // extern "C"

namespace msa {

msa_status plan_config(const msa_decode_shape* shape, bool prefill, int32_t real_rows,
                       int device, bool allow_fused, msa_plan_s* plan) {
  const bool dense = shape->topk_blocks == 0;
  if (dense && prefill)
    return fail(MSA_ERR_UNSUPPORTED, "a prefill plan needs top-k selections (topk_blocks >= 1)");
  if (shape->topk_blocks < 0)
    return fail(MSA_ERR_INVALID_ARG, "topk_blocks must be >= 1, or 0 for dense decode (got %d)",
                shape->topk_blocks);
  if (shape->topk_blocks > msa::kMaxTopk)
    return fail(MSA_ERR_UNSUPPORTED, "topk_blocks %d exceeds %d", shape->topk_blocks,
                msa::kMaxTopk);
  if (shape->num_splits < 0 || shape->num_splits > msa::kMaxSplits)
    return fail(MSA_ERR_INVALID_ARG, "num_splits must be 0 (auto) or 1..%d (got %d)",
                msa::kMaxSplits, shape->num_splits);
  if (device < 0) return fail(MSA_ERR_INVALID_ARG, "device must be >= 0 (got %d)", device);

  const int32_t num_rows = shape->num_token_rows ? shape->num_token_rows : real_rows;
  int32_t tile_rows = 1;
  int64_t units = 0;
  msa_status st = choose_tiles(shape, prefill, dense, num_rows, &tile_rows, &units);
  if (st != MSA_OK) return st;
  if (units > INT32_MAX) return fail(MSA_ERR_UNSUPPORTED, "launch grid too large");
  const int32_t splits = choose_splits(shape, units, dense);
  const int64_t grid =
      (tile_rows == 1 ? msa::xcd_groups(units, shape->num_kv_heads)
       : (dense || tile_rows == 8)
           ? (units + msa::kXcdSlots - 1) / msa::kXcdSlots
           : msa::tile_block_groups(units / shape->num_kv_heads, shape->num_kv_heads)) *
      msa::kXcdSlots * splits;
  if (grid > INT32_MAX) return fail(MSA_ERR_UNSUPPORTED, "launch grid too large");
  const int64_t per_row = (int64_t)shape->num_q_heads * splits;
  const int64_t o_bytes = splits > 1 ? (int64_t)num_rows * per_row * msa::kHeadDim * 4 : 0;
  const int64_t ml_bytes = splits > 1 ? (int64_t)num_rows * per_row * 2 * 4 : 0;
  // The single-row attend merges 2..4 splits itself (the last split of a unit
  // to finish combines them); other plans launch the merge kernel.
  const bool fused =
      allow_fused && tile_rows == 1 && splits > 1 && splits <= msa::kMaxFusedSplits;
  const int64_t arrival_bytes = fused ? (units * 4 + 255) / 256 * 256 : 0;

  *plan = msa_plan_s{};
  plan->shape = *shape;
  plan->prefill = prefill;
  plan->dense = dense;
  plan->tile_rows = tile_rows;
  plan->num_units = (int32_t)units;
  plan->shape.num_token_rows = num_rows;
  plan->shape.num_splits = splits;
  plan->shape.tile_rows = tile_rows;
  plan->device = device;
  plan->splits = splits;
  plan->real_rows = real_rows;
  plan->num_rows = num_rows;
  plan->fused = fused;
  plan->arrival_bytes = arrival_bytes;
  plan->o_bytes = o_bytes;
  plan->arena_bytes = arrival_bytes + o_bytes + ml_bytes;
  return ok();
}

}  // namespace msa

extern "C" {

static msa_status make_plan(const msa_decode_shape* shape, bool prefill, int32_t real_rows,
                            int device, msa_plan* plan_out) {
  msa_plan_s cfg;
  msa_status st = msa::plan_config(shape, prefill, real_rows, device, true, &cfg);
  if (st != MSA_OK) return st;
  msa_plan plan = new (std::nothrow) msa_plan_s(cfg);
  if (plan == nullptr) return fail(MSA_ERR_OUT_OF_MEMORY, "host allocation failed");
  if (plan->arena_bytes > 0) {
    // The arena is the plan's only device state; a plan without one makes no
    // HIP call here.
    DeviceGuard guard;
    hipError_t e = guard.enter(device);
    if (e != hipSuccess) {
      delete plan;
      return device_fail(e, "hipSetDevice");
    }
    e = hipMalloc(&plan->arena, (size_t)plan->arena_bytes);
    if (e != hipSuccess) {
      const long long bytes = (long long)plan->arena_bytes;
      delete plan;
      if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
        return fail(MSA_ERR_OUT_OF_MEMORY, "partial arena of %lld bytes: %s", bytes,
                    hipGetErrorString(e));
      return device_fail(e, "hipMalloc");
    }
    char* base = static_cast<char*>(plan->arena);
    if (plan->fused) {
      // Counters start at zero; every fused run leaves them at zero.
      plan->arrivals = reinterpret_cast<int32_t*>(base);
      e = hipMemset(plan->arrivals, 0, (size_t)plan->arrival_bytes);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) {
        (void)hipFree(plan->arena);
        delete plan;
        return device_fail(e, "arrival counter initialisation");
      }
      base += plan->arrival_bytes;
    }
    plan->part_o = reinterpret_cast<float*>(base);
    plan->part_ml = reinterpret_cast<float*>(base + plan->o_bytes);
  }
  *plan_out = plan;
  return ok();
}

msa_status msa_sparse_decode_plan_destroy(msa_plan plan) {
  if (plan == nullptr) return ok();
  msa_status st = MSA_OK;
  if (plan->arena != nullptr) {
    DeviceGuard guard;
    hipError_t e = guard.enter(plan->device);
    if (e == hipSuccess) e = hipFree(plan->arena);
    if (e != hipSuccess) st = device_fail(e, "hipFree");
  }
  delete plan;
  return st == MSA_OK ? ok() : st;
}

msa_status msa_sparse_decode_plan_info(msa_plan plan, int32_t* num_splits, int64_t* arena_bytes,
                                       msa_decode_shape* shape_out) {
  if (plan == nullptr) return fail(MSA_ERR_INVALID_ARG, "plan is NULL");
  if (num_splits) *num_splits = plan->splits;
  if (arena_bytes) *arena_bytes = plan->arena_bytes;
  if (shape_out) *shape_out = plan->shape;
  return ok();
}

// seq_lens is the decode position source; cu_q / ctx the prefill one (a
// prefill plan passes seq_lens = NULL).
}  // extern "C"

namespace msa {

msa_status run_plan(const msa_plan_s* plan, const void* q, const void* kv_cache,
                    const int64_t kv_strides[4], int64_t num_kv_blocks, float q_scale,
                    float k_scale, float v_scale, const int32_t* block_table,
                    const int32_t* seq_lens, const int32_t* cu_q, const int32_t* ctx,
                    const int32_t* topk, const int64_t topk_strides[3], void* out,
                    float sm_scale, void* stream, bool merge, const SelectSource* sel) {
  if (plan == nullptr) return fail(MSA_ERR_INVALID_ARG, "plan is NULL");
  const msa_decode_shape& s = plan->shape;
  if (q == nullptr || out == nullptr) return fail(MSA_ERR_INVALID_ARG, "q and out must be non-NULL");
  if (!aligned16(q) || !aligned16(out))
    return fail(MSA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (plan->prefill) {
    if (block_table == nullptr || cu_q == nullptr || ctx == nullptr || topk == nullptr)
      return fail(MSA_ERR_INVALID_ARG,
                  "block_table, cu_seqlens_q, context_lens and topk must be non-NULL");
  } else if (block_table == nullptr || seq_lens == nullptr) {
    return fail(MSA_ERR_INVALID_ARG, "block_table and seq_lens must be non-NULL");
  } else if (sel != nullptr) {
    if (plan->dense || plan->tile_rows != 1)
      return fail(MSA_ERR_UNSUPPORTED,
                  "the selecting attend runs on single-row sparse decode plans (tile_rows 1)");
  } else if (plan->dense != (topk == nullptr)) {
    return fail(MSA_ERR_INVALID_ARG, plan->dense ? "a dense plan takes topk = NULL"
                                                 : "block_table, seq_lens and topk must be "
                                                   "non-NULL");
  }
  if (!plan->dense && sel == nullptr) {
    if (topk_strides == nullptr) return fail(MSA_ERR_INVALID_ARG, "topk_strides is NULL");
    for (int d = 0; d < 3; ++d)
      if (topk_strides[d] < 0) return fail(MSA_ERR_INVALID_ARG, "topk strides must be >= 0");
  }
  msa_status st = check_kv(kv_cache, kv_strides, num_kv_blocks, s.kv_dtype);
  if (st != MSA_OK) return st;
  st = check_scales(q_scale, k_scale);
  if (st != MSA_OK) return st;
  if (!std::isfinite(v_scale) || !std::isfinite(sm_scale))
    return fail(MSA_ERR_INVALID_ARG, "scales must be finite");
  if (!(sm_scale > 0.f)) return fail(MSA_ERR_INVALID_ARG, "sm_scale must be positive");

  const int64_t eb = elem_bytes(s.kv_dtype);
  msa::AttendParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.kv_s0 = kv_strides[0] * eb;
  p.kv_s1 = kv_strides[1] * eb;
  p.kv_s2 = kv_strides[2] * eb;
  p.num_kv_blocks = num_kv_blocks;
  p.block_table = block_table;
  p.bt_stride = s.page_table_stride;
  p.seq_lens = seq_lens;
  p.topk = topk;
  if (sel != nullptr) {
    p.sel_score = sel->score;
    p.sel_s0 = sel->s0;
    p.sel_s1 = sel->s1;
    p.sel_s2 = sel->s2;
    p.sel_max_blocks = sel->max_blocks;
    p.sel_topk_out = sel->topk_out;
  } else if (!plan->dense) {
    p.tk_s0 = topk_strides[0];
    p.tk_s1 = topk_strides[1];
    p.tk_s2 = topk_strides[2];
  }
  p.out = static_cast<uint16_t*>(out);
  p.part_o = plan->part_o;
  p.part_ml = plan->part_ml;
  p.scale_log2 =
      (float)((double)sm_scale * (double)q_scale * (double)k_scale * 1.4426950408889634);
  p.v_scale = v_scale;
  p.dql = s.decode_query_len;
  p.real_rows = plan->real_rows;
  p.num_rows = plan->num_rows;
  p.hq = s.num_q_heads;
  p.hkv = s.num_kv_heads;
  p.group = s.num_q_heads / s.num_kv_heads;
  p.topk_k = s.topk_blocks;
  p.splits = plan->splits;
  p.num_units = plan->num_units;
  p.tile_dense = plan->dense ? 1 : 0;
  // Longest request first for sparse decode tiles (2 or 4 rows) of a small
  // batch whose tiles never span two requests.
  p.len_order = (!plan->prefill && !plan->dense && (plan->tile_rows == 2 || plan->tile_rows == 4) &&
                 s.batch <= 64 && s.decode_query_len % plan->tile_rows == 0)
                    ? 1
                    : 0;
  p.arrivals = plan->fused ? plan->arrivals : nullptr;
  if (plan->prefill) {
    p.cu_q = cu_q;
    p.ctx_lens = ctx;
    p.num_reqs = s.batch;
    p.dql = 1;
    p.real_rows = plan->num_rows;
  }

  DeviceGuard guard;
  hipError_t e = guard.enter(plan->device);
  if (e != hipSuccess) return device_fail(e, "hipSetDevice");
  hipStream_t st_ = static_cast<hipStream_t>(stream);
  // 8-row tiles (8-bit caches only) stage pages through LDS; 2- and 4-row
  // tiles keep them in registers.
  if (plan->tile_rows == 8)
    e = msa::launch_union(p, s.kv_dtype, s.q_dtype, plan->tile_rows, st_);
  else if (plan->tile_rows > 1)
    e = msa::launch_tile(p, s.kv_dtype, s.q_dtype, plan->tile_rows, st_);
  else
    e = msa::launch_attend(p, s.kv_dtype, s.q_dtype, st_);
  if (e != hipSuccess) return device_fail(e, "attend launch");
  if (merge && plan->splits > 1 && !plan->fused) {
    e = msa::launch_merge(p, st_);
    if (e != hipSuccess) return device_fail(e, "merge launch");
  }
  return ok();
}

}  // namespace msa

extern "C" {

msa_status msa_sparse_decode_run(msa_plan plan, const void* q, const void* kv_cache,
                                 const int64_t kv_strides[4], int64_t num_kv_blocks,
                                 float q_scale, float k_scale, float v_scale,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* topk, const int64_t topk_strides[3], void* out,
                                 float sm_scale, void* stream) {
  if (plan != nullptr && plan->prefill)
    return fail(MSA_ERR_INVALID_ARG, "a prefill plan runs through msa_sparse_prefill_run");
  return msa::run_plan(plan, q, kv_cache, kv_strides, num_kv_blocks, q_scale, k_scale, v_scale,
                    block_table, seq_lens, nullptr, nullptr, topk, topk_strides, out, sm_scale,
                    stream, true);
}

msa_status msa_sparse_prefill_run(msa_plan plan, const void* q, const void* kv_cache,
                                  const int64_t kv_strides[4], int64_t num_kv_blocks,
                                  float q_scale, float k_scale, float v_scale,
                                  const int32_t* block_table, const int32_t* cu_seqlens_q,
                                  const int32_t* context_lens, const int32_t* topk,
                                  const int64_t topk_strides[3], void* out, float sm_scale,
                                  void* stream) {
  if (plan != nullptr && !plan->prefill)
    return fail(MSA_ERR_INVALID_ARG, "a decode plan runs through msa_sparse_decode_run");
  return msa::run_plan(plan, q, kv_cache, kv_strides, num_kv_blocks, q_scale, k_scale, v_scale,
                    block_table, nullptr, cu_seqlens_q, context_lens, topk, topk_strides, out,
                    sm_scale, stream, true);
}

msa_status msa_sparse_decode_attend(msa_plan plan, const void* q, const void* kv_cache,
                                    const int64_t kv_strides[4], int64_t num_kv_blocks,
                                    float q_scale, float k_scale, float v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* topk, const int64_t topk_strides[3],
                                    void* out, float sm_scale, void* stream) {
  if (plan != nullptr && plan->prefill)
    return fail(MSA_ERR_INVALID_ARG, "a prefill plan runs through msa_sparse_prefill_run");
  return msa::run_plan(plan, q, kv_cache, kv_strides, num_kv_blocks, q_scale, k_scale, v_scale,
                    block_table, seq_lens, nullptr, nullptr, topk, topk_strides, out, sm_scale,
                    stream, false);
}

msa_status msa_sparse_decode_select_run(msa_plan plan, const void* q, const void* kv_cache,
                                        const int64_t kv_strides[4], int64_t num_kv_blocks,
                                        float q_scale, float k_scale, float v_scale,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* score, const int64_t score_strides[3],
                                        int32_t max_blocks, int32_t* topk_out, void* out,
                                        float sm_scale, void* stream) {
  if (plan != nullptr && plan->prefill)
    return fail(MSA_ERR_INVALID_ARG, "a prefill plan runs through msa_sparse_prefill_run");
  if (score == nullptr) return fail(MSA_ERR_INVALID_ARG, "score must be non-NULL");
  if (score_strides == nullptr) return fail(MSA_ERR_INVALID_ARG, "score_strides is NULL");
  for (int d = 0; d < 3; ++d)
    if (score_strides[d] < 0) return fail(MSA_ERR_INVALID_ARG, "score strides must be >= 0");
  if (max_blocks < 1 || max_blocks > msa::kMaxScoreBlocks)
    return fail(MSA_ERR_INVALID_ARG, "max_blocks must be in 1..%d (got %d)",
                msa::kMaxScoreBlocks, max_blocks);
  const msa::SelectSource sel{score, score_strides[0], score_strides[1], score_strides[2],
                              max_blocks, topk_out};
  return msa::run_plan(plan, q, kv_cache, kv_strides, num_kv_blocks, q_scale, k_scale, v_scale,
                       block_table, seq_lens, nullptr, nullptr, nullptr, nullptr, out, sm_scale,
                       stream, true, &sel);
}

msa_status msa_sparse_decode_merge(msa_plan plan, void* out, float v_scale, void* stream) {
  if (plan == nullptr) return fail(MSA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->prefill)
    return fail(MSA_ERR_INVALID_ARG, "a prefill plan runs through msa_sparse_prefill_run");
  if (out == nullptr || !aligned16(out))
    return fail(MSA_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
  if (!std::isfinite(v_scale)) return fail(MSA_ERR_INVALID_ARG, "scales must be finite");
  if (plan->splits == 1 || plan->fused) return ok();
  const msa_decode_shape& s = plan->shape;
  msa::AttendParams p{};
  p.out = static_cast<uint16_t*>(out);
  p.part_o = plan->part_o;
  p.part_ml = plan->part_ml;
  p.v_scale = v_scale;
  p.dql = s.decode_query_len;
  p.real_rows = plan->real_rows;
  p.num_rows = plan->num_rows;
  p.hq = s.num_q_heads;
  p.hkv = s.num_kv_heads;
  p.group = s.num_q_heads / s.num_kv_heads;
  p.topk_k = s.topk_blocks;
  p.splits = plan->splits;
  p.num_units = plan->num_rows * s.num_kv_heads;
  DeviceGuard guard;
  hipError_t e = guard.enter(plan->device);
  if (e != hipSuccess) return device_fail(e, "hipSetDevice");
  e = msa::launch_merge(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "merge launch");
  return ok();
}

msa_status msa_topk_select(const float* score, const int64_t score_strides[3],
                           int32_t num_kv_heads, int32_t max_blocks, int32_t num_rows,
                           int32_t* topk_out, int32_t topk_k, void* stream) {
  if (score == nullptr || topk_out == nullptr)
    return fail(MSA_ERR_INVALID_ARG, "score and topk_out must be non-NULL");
  if (score_strides == nullptr) return fail(MSA_ERR_INVALID_ARG, "score_strides is NULL");
  for (int d = 0; d < 3; ++d)
    if (score_strides[d] < 0) return fail(MSA_ERR_INVALID_ARG, "score strides must be >= 0");
  if (num_kv_heads < 1 || num_rows < 1)
    return fail(MSA_ERR_INVALID_ARG, "num_kv_heads and num_rows must be >= 1");
  if (max_blocks < 1 || max_blocks > msa::kMaxScoreBlocks)
    return fail(MSA_ERR_INVALID_ARG, "max_blocks must be in 1..%d (got %d)",
                msa::kMaxScoreBlocks, max_blocks);
  if (topk_k < 1 || topk_k > msa::kMaxTopk)
    return fail(MSA_ERR_INVALID_ARG, "topk_k must be in 1..%d (got %d)", msa::kMaxTopk, topk_k);
  if ((int64_t)num_rows * num_kv_heads > INT32_MAX)
    return fail(MSA_ERR_UNSUPPORTED, "launch grid too large");
  msa::SelectParams p{};
  p.score = score;
  p.sc_s0 = score_strides[0];
  p.sc_s1 = score_strides[1];
  p.sc_s2 = score_strides[2];
  p.topk_out = topk_out;
  p.hkv = num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_rows = num_rows;
  p.k = topk_k;
  hipError_t e = msa::launch_select(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "select launch");
  return ok();
}

msa_status msa_block_score_topk(const msa_decode_shape* shape, const void* q,
                                const void* kv_cache, const int64_t kv_strides[4],
                                int64_t num_kv_blocks, float q_scale, float k_scale,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_blocks, float* score,
                                const int64_t score_strides[3], int32_t* topk_out,
                                int32_t topk_k, void* stream) {
  msa_status st = check_common_shape(shape);
  if (st != MSA_OK) return st;
  if (q == nullptr || !aligned16(q)) return fail(MSA_ERR_INVALID_ARG, "q must be non-NULL and 16-byte aligned");
  if (block_table == nullptr || seq_lens == nullptr)
    return fail(MSA_ERR_INVALID_ARG, "block_table and seq_lens must be non-NULL");
  if (score == nullptr) return fail(MSA_ERR_INVALID_ARG, "score must be non-NULL");
  if (score_strides == nullptr) return fail(MSA_ERR_INVALID_ARG, "score_strides is NULL");
  for (int d = 0; d < 3; ++d)
    if (score_strides[d] < 0) return fail(MSA_ERR_INVALID_ARG, "score strides must be >= 0");
  st = check_kv(kv_cache, kv_strides, num_kv_blocks, shape->kv_dtype);
  if (st != MSA_OK) return st;
  if (max_blocks < 1 || max_blocks > msa::kMaxScoreBlocks)
    return fail(MSA_ERR_INVALID_ARG, "max_blocks must be in 1..%d (got %d)",
                msa::kMaxScoreBlocks, max_blocks);
  if (topk_out != nullptr && (topk_k < 1 || topk_k > msa::kMaxTopk))
    return fail(MSA_ERR_INVALID_ARG, "topk_k must be in 1..%d (got %d)", msa::kMaxTopk, topk_k);
  st = check_scales(q_scale, k_scale);
  if (st != MSA_OK) return st;
  if (shape->batch > msa::kMaxScoreBatch)
    return fail(MSA_ERR_UNSUPPORTED, "the scorer supports batch <= %d (got %d)",
                msa::kMaxScoreBatch, shape->batch);

  const int32_t real_rows = shape->batch * shape->decode_query_len;
  const int32_t num_rows = shape->num_token_rows ? shape->num_token_rows : real_rows;
  const int64_t eb = elem_bytes(shape->kv_dtype);
  msa::ScoreParams p{};
  p.q = static_cast<const uint8_t*>(q);
  p.kv = static_cast<const uint8_t*>(kv_cache);
  p.kv_s0 = kv_strides[0] * eb;
  p.kv_s1 = kv_strides[1] * eb;
  p.kv_s2 = kv_strides[2] * eb;
  p.num_kv_blocks = num_kv_blocks;
  p.block_table = block_table;
  p.bt_stride = shape->page_table_stride;
  p.seq_lens = seq_lens;
  p.score = score;
  p.sc_s0 = score_strides[0];
  p.sc_s1 = score_strides[1];
  p.sc_s2 = score_strides[2];
  p.qk_scale = (float)((double)q_scale * (double)k_scale);
  p.batch = shape->batch;
  p.dql = shape->decode_query_len;
  p.real_rows = real_rows;
  p.num_rows = num_rows;
  p.hq = shape->num_q_heads;
  p.hkv = shape->num_kv_heads;
  p.group = shape->num_q_heads / shape->num_kv_heads;
  p.max_blocks = max_blocks;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_score(p, shape->kv_dtype, shape->q_dtype, hs);
  if (e != hipSuccess) return device_fail(e, "score launch");
  if (topk_out == nullptr) return ok();  // scores only (msa_sparse_decode_select_run selects)
  return msa_topk_select(score, score_strides, shape->num_kv_heads, max_blocks, num_rows,
                         topk_out, topk_k, stream);
}

static msa_status fp8_to_bf16(const void* in, void* out, int64_t n, int fmt, void* stream) {
  if (in == nullptr || out == nullptr) return fail(MSA_ERR_INVALID_ARG, "in and out must be non-NULL");
  if (n < 1 || n > ((int64_t)1 << 40)) return fail(MSA_ERR_INVALID_ARG, "n out of range");
  hipError_t e = msa::launch_fp8_to_bf16(static_cast<const uint8_t*>(in),
                                         static_cast<uint16_t*>(out), n, fmt,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "fp8 conversion launch");
  return ok();
}

msa_status msa_probe_read_runs(const void* base, int64_t buffer_bytes,
                               const int64_t* run_offsets, const int32_t* run_bytes,
                               int32_t num_runs, const int32_t* wg_first_run,
                               int32_t num_workgroups, uint32_t* out, void* stream) {
  if (num_workgroups < 0) return fail(MSA_ERR_INVALID_ARG, "num_workgroups must be >= 0");
  if (num_workgroups > (1 << 24)) return fail(MSA_ERR_UNSUPPORTED, "num_workgroups exceeds 2^24");
  if (num_runs < 0) return fail(MSA_ERR_INVALID_ARG, "num_runs must be >= 0");
  if (num_workgroups == 0) return ok();
  if (base == nullptr || wg_first_run == nullptr || out == nullptr)
    return fail(MSA_ERR_INVALID_ARG, "base, wg_first_run and out must be non-NULL");
  if (num_runs > 0 && (run_offsets == nullptr || run_bytes == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "run_offsets and run_bytes must be non-NULL");
  if (!aligned16(base)) return fail(MSA_ERR_INVALID_ARG, "base is not 16-byte aligned");
  if (buffer_bytes < 16) return fail(MSA_ERR_INVALID_ARG, "buffer_bytes must be >= 16");
  hipError_t e = msa::launch_read_runs(
      static_cast<const uint8_t*>(base), buffer_bytes, run_offsets, run_bytes, wg_first_run,
      num_runs, num_workgroups, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "read-runs probe launch");
  return ok();
}

msa_status msa_fp8_e4m3_to_bf16(const void* in, void* out, int64_t n, void* stream) {
  return fp8_to_bf16(in, out, n, msa::kKvE4m3, stream);
}

msa_status msa_fp8_e5m2_to_bf16(const void* in, void* out, int64_t n, void* stream) {
  return fp8_to_bf16(in, out, n, msa::kKvE5m2, stream);
}

msa_status msa_mxfp4_to_bf16(const void* kv_cache, const int64_t kv_strides[4],
                             int64_t num_kv_blocks, int32_t num_kv_heads, void* out,
                             void* stream) {
  msa_status st = check_kv(kv_cache, kv_strides, num_kv_blocks, MSA_KV_MXFP4);
  if (st != MSA_OK) return st;
  if (out == nullptr) return fail(MSA_ERR_INVALID_ARG, "out is NULL");
  if (!aligned16(out)) return fail(MSA_ERR_INVALID_ARG, "out is not 16-byte aligned");
  if (num_kv_heads < 1 || num_kv_heads > 1024)
    return fail(MSA_ERR_INVALID_ARG, "num_kv_heads must be in 1..1024 (got %d)", num_kv_heads);
  if (num_kv_blocks * num_kv_heads * msa::kPage * 8 > ((int64_t)1 << 39))
    return fail(MSA_ERR_UNSUPPORTED, "cache too large for one conversion launch");
  hipError_t e = msa::launch_mxfp4_to_bf16(static_cast<const uint8_t*>(kv_cache), kv_strides[0],
                                           kv_strides[1], kv_strides[2], num_kv_blocks,
                                           num_kv_heads, static_cast<uint16_t*>(out),
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "MXFP4 conversion launch");
  return ok();
}

}  // extern "C"
