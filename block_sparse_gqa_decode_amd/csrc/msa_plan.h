// Host-side plan state and the internal entry points the C-ABI translation
// units share (msa_api.cpp, msa_noalloc.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_sparse_decode.h"

// One plan: a validated static shape and its launch configuration, plus the
// fp32 split-K partial arena the kernels write (the library's allocation for
// a plan, or caller-free static scratch for the no-allocation entry point).
struct msa_plan_s {
  msa_decode_shape shape;   // for a prefill plan: decode_query_len = 0
  bool prefill;
  bool dense;               // every visible block (topk_blocks == 0)
  int32_t tile_rows;        // 1: one row per workgroup; 2 / 4: multi-row tiles
  int32_t num_units;        // workgroups per split
  int device;
  int32_t splits;
  int32_t real_rows;
  int32_t num_rows;
  bool fused;               // splits merged inside the attend (2..4 splits, 1 row)
  int64_t arrival_bytes;    // arena bytes of the fused merge's arrival counters
  int64_t o_bytes;          // arena bytes of the fp32 partial O
  int64_t arena_bytes;      // arrival_bytes + o_bytes + the (max, sum) partials
  void* arena;              // owned by the plan (null when arena_bytes == 0 or
                            // when the arena is not the plan's)
  float* part_o;
  float* part_ml;
  int32_t* arrivals;        // per-unit arrival counters of the fused merge
};

namespace msa {

// Record a non-OK status and its message for msa_last_error(); returns s.
msa_status fail(msa_status s, const char* fmt, ...);
// Clear the message; returns MSA_OK.
msa_status ok();

// The checks every decode shape passes (plan and indexer entry points).
msa_status check_common_shape(const msa_decode_shape* s);

// Validate a (decode or prefill) shape and fill `plan` with its launch
// configuration and arena layout, without allocating or calling HIP; the
// arena pointers are left null.  allow_fused = false keeps a plan with 2..4
// single-row splits on the separate merge kernel (no arrival counters).
msa_status plan_config(const msa_decode_shape* shape, bool prefill, int32_t real_rows,
                       int device, bool allow_fused, msa_plan_s* plan);

// The block scores a single-row decode attend selects its own top-k from
// (msa_sparse_decode_select_run); topk_out may be null.
struct SelectSource {
  const float* score;
  int64_t s0, s1, s2;
  int32_t max_blocks;
  int32_t* topk_out;
};

// One decode or prefill run of a configured plan whose arena pointers are set
// (seq_lens for decode, cu_q / ctx for prefill); `merge` false launches the
// attend alone.  With `sel`, topk is NULL and the attend selects each row's
// top-k from the scores itself.  Validates every run argument before any HIP
// call.
msa_status run_plan(const msa_plan_s* plan, const void* q, const void* kv_cache,
                    const int64_t kv_strides[4], int64_t num_kv_blocks, float q_scale,
                    float k_scale, float v_scale, const int32_t* block_table,
                    const int32_t* seq_lens, const int32_t* cu_q, const int32_t* ctx,
                    const int32_t* topk, const int64_t topk_strides[3], void* out,
                    float sm_scale, void* stream, bool merge,
                    const SelectSource* sel = nullptr);

// Makes `dev` the current HIP device for the guard's lifetime.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t enter(int dev) {
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != dev) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return e;
      changed = true;
    }
    return hipSuccess;
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

}  // namespace msa
