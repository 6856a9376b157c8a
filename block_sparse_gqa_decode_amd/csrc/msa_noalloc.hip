// msa_sparse_decode_run_noalloc: the decode step of msa_sparse_decode_run for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  It takes the
// static shape instead of a plan, configures the launch exactly as a plan
// would (host arithmetic only), and puts the fp32 split-K partials in a
// file-scope device array instead of a plan's arena.
//
// The array: `scratch` below, kNoAllocScratchBytes per device, held by every
// GPU the library runs on until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the first call on each device, with that device current, looks
// up the device's own copy with hipGetSymbolAddress and keeps that pointer,
// and kernels receive only it.
//
// What stays valid between calls: nothing needs to.  Splits are merged by the
// separate merge kernel (never the in-attend merge, whose arrival counters
// would have to start at zero), every split of every real token row writes
// its whole partial before the merge reads it, and padding rows are neither
// written nor read.  So the array's earlier contents never reach an output.
// Every call on a device shares that device's array: calls that overlap on
// one GPU (two streams, or two host threads) race and must be serialized.
#include <mutex>

#include "msa_internal.h"
#include "msa_plan.h"
#include "msa_sparse_decode.h"

namespace {

constexpr int64_t kNoAllocScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The device address of `scratch` on `device`, looked up once per device.
msa_status scratch_on(int device, void** out) {
  if (device < 0 || device >= kMaxDevices)
    return msa::fail(MSA_ERR_INVALID_ARG, "device must be in 0..%d (got %d)", kMaxDevices - 1,
                     device);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    msa::DeviceGuard guard;
    hipError_t e = guard.enter(device);
    if (e != hipSuccess)
      return msa::fail(MSA_ERR_DEVICE, "hipSetDevice failed: %s", hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return msa::fail(MSA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s",
                       hipGetErrorString(e));
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return MSA_OK;
}

}  // namespace

extern "C" msa_status msa_sparse_decode_run_noalloc(
    const msa_decode_shape* shape, int device, const void* q, const void* kv_cache,
    const int64_t kv_strides[4], int64_t num_kv_blocks, float q_scale, float k_scale,
    float v_scale, const int32_t* block_table, const int32_t* seq_lens, const int32_t* topk,
    const int64_t topk_strides[3], void* out, float sm_scale, void* stream) {
  msa_status st = msa::check_common_shape(shape);
  if (st != MSA_OK) return st;
  msa_plan_s plan;
  st = msa::plan_config(shape, false, shape->batch * shape->decode_query_len, device,
                        /*allow_fused=*/false, &plan);
  if (st != MSA_OK) return st;
  if (plan.arena_bytes > kNoAllocScratchBytes)
    return msa::fail(MSA_ERR_UNSUPPORTED,
                     "this shape needs %lld bytes of split partials (%d splits), above the "
                     "%lld-byte static scratch of the no-allocation entry point; use fewer "
                     "splits or a plan",
                     (long long)plan.arena_bytes, plan.splits, (long long)kNoAllocScratchBytes);
  if (plan.arena_bytes > 0) {
    void* base = nullptr;
    st = scratch_on(device, &base);
    if (st != MSA_OK) return st;
    plan.part_o = static_cast<float*>(base);
    plan.part_ml = reinterpret_cast<float*>(static_cast<char*>(base) + plan.o_bytes);
  }
  return msa::run_plan(&plan, q, kv_cache, kv_strides, num_kv_blocks, q_scale, k_scale,
                       v_scale, block_table, seq_lens, nullptr, nullptr, topk, topk_strides, out,
                       sm_scale, stream, true);
}
