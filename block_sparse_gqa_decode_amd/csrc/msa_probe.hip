// Memory-rate probe for gfx950: reads byte runs of a device buffer and does
// nothing else with them.
//
// The decode attend's time on short steps is partly data movement (the live
// K|V rows of the selected pages) and partly fixed cost (resolving the top-k
// row through the block table, the softmax and MFMA work, the split merge).
// Fed the attend's own page rows, dealt to the same workgroup ids, this
// kernel measures the first part alone: the rate at which this part gathers
// exactly those bytes.  Fed contiguous runs of the same sizes, it measures a
// plain streaming read.
//
// Each workgroup of 256 threads walks its runs in order.  One pass of the
// workgroup reads 4 KiB of a run as fully coalesced 16-byte loads (thread i
// takes bytes 16i..16i+15 of each 4 KiB), so a run of up to 32 KiB is eight
// loads per thread.  Two runs are in flight per workgroup: the loads of the
// next run are issued before the current one is consumed, as a ring unrolled
// twice so every register index is static.  Loads are unconditional: bytes
// past a run's end re-read its last 16 bytes (cache hits) and are not
// counted, and the ring's tail re-reads the last run.  The workgroup's
// result is the XOR of every 32-bit word of its runs, which the host can
// recompute exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;                          // 16-byte loads per thread per run
constexpr int kPass = kThreads * 16;               // bytes one pass of the workgroup reads
constexpr int kMaxRun = kPass * kLoads;            // 32 KiB
constexpr int kMaxRunsPerWg = 512;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Run {
  const uint8_t* ptr;   // start of the run (a valid address even for a skipped run)
  int len;              // bytes to count; 0 for a skipped run
};

__device__ __forceinline__ void issue(u32x4 (&r)[kLoads], const Run& run, int tid) {
  const int last = (run.len > 16 ? run.len : 16) - 16;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int off = min(tid * 16 + j * kPass, last);
    r[j] = *reinterpret_cast<const u32x4*>(run.ptr + off);
  }
}

__device__ __forceinline__ uint32_t consume(const u32x4 (&r)[kLoads], int len, int tid) {
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool in = tid * 16 + j * kPass < len;
    const uint32_t v = r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    x ^= in ? v : 0u;
  }
  return x;
}

__global__ __launch_bounds__(kThreads) void read_runs_kernel(
    const uint8_t* __restrict__ base, int64_t buffer_bytes,
    const int64_t* __restrict__ run_off, const int32_t* __restrict__ run_len,
    const int32_t* __restrict__ wg_first, int32_t num_runs, uint32_t* __restrict__ out) {
  __shared__ int64_t s_off[kMaxRunsPerWg];
  __shared__ int32_t s_len[kMaxRunsPerWg];
  __shared__ uint32_t s_x[kThreads / 64];
  __shared__ int32_t s_bad;

  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  // The run range comes from caller memory: clamp it into [0, num_runs].
  const int first = min(max(wg_first[w], 0), num_runs);
  const int last = min(max(wg_first[w + 1], first), num_runs);
  int n = last - first;
  int bad = 0;
  if (n > kMaxRunsPerWg) {
    bad = n - kMaxRunsPerWg;
    n = kMaxRunsPerWg;
  }
  if (tid == 0) s_bad = bad;
  __syncthreads();
  // A run outside the buffer, misaligned, empty or longer than 32 KiB is
  // skipped (read nothing) and counted.
  for (int i = tid; i < n; i += kThreads) {
    int64_t o = run_off[first + i];
    int32_t l = run_len[first + i];
    const bool ok = o >= 0 && l >= 16 && l <= kMaxRun && (l & 15) == 0 && (o & 15) == 0 &&
                    o <= buffer_bytes - l;
    if (!ok) {
      atomicAdd(&s_bad, 1);
      o = 0;
      l = 0;
    }
    s_off[i] = o;
    s_len[i] = l;
  }
  __syncthreads();

  uint32_t acc = 0;
  if (n > 0) {
    u32x4 a[kLoads], b[kLoads];
    auto run_at = [&](int i) {
      const int64_t o = s_off[i];
      return Run{base + o, s_len[i]};
    };
    Run ra = run_at(0);
    issue(a, ra, tid);
    // The scheduling barriers keep each run's loads ahead of the previous
    // run's use; without them the scheduler moves that use, and its waits,
    // in front of the loads.  The use of b is unconditional for the same
    // reason (a branch would take b's loads with it).
    for (int i = 0; i < n; i += 2) {
      const Run rb = run_at(min(i + 1, n - 1));
      issue(b, rb, tid);
      __builtin_amdgcn_sched_barrier(0);
      acc ^= consume(a, ra.len, tid);
      ra = run_at(min(i + 2, n - 1));
      issue(a, ra, tid);
      __builtin_amdgcn_sched_barrier(0);
      acc ^= consume(b, i + 1 < n ? rb.len : 0, tid);
    }
  }

  // XOR over the workgroup: within each wavefront by lane shuffles, then
  // across the four wavefronts through LDS.
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m);
  if ((tid & 63) == 0) s_x[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int v = 0; v < kThreads / 64; ++v) x ^= s_x[v];
    out[2 * w] = x;
    out[2 * w + 1] = (uint32_t)s_bad;
  }
}

}  // namespace

hipError_t launch_read_runs(const uint8_t* base, int64_t buffer_bytes, const int64_t* run_off,
                            const int32_t* run_len, const int32_t* wg_first, int32_t num_runs,
                            int32_t num_workgroups, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_runs_kernel, dim3(num_workgroups), dim3(kThreads), 0, stream, base,
                     buffer_bytes, run_off, run_len, wg_first, num_runs, out);
  return hipGetLastError();
}

}  // namespace msa
