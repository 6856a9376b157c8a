// Device-side mapping of a token row to its request and position, shared by
// the single-row and multi-row attend kernels.
#pragma once

#include "msa_internal.h"

namespace msa {

// The request of token row t and the token's position, or false for a
// padding row.  A decode row t belongs to request t / dql at position
// seq_len - dql + t % dql (vLLM test file
// test_minimax_m3_msa_cutlass_sparse_decode.py, _make_topk); a ragged prefill
// row belongs to the request r with cu_q[r] <= t < cu_q[r+1] at position
// ctx_lens[r] + t - cu_q[r] (vLLM API page
// "vllm.models.minimax_m3.common.sparse_attention",
// MiniMaxM3SparsePrefillMetadata).  The lookup is a binary search, so r stays
// in [0, num_reqs) whatever the device data holds.
// kVarlen selects the form at compile time (false: decode rows, true: ragged
// prefill rows) so a decode kernel carries no prefill code; the default reads
// the form from the parameters.
template <int kVarlen = -1>
__device__ __forceinline__ bool locate_token(const AttendParams& p, int t, int& r, int& pos) {
  const bool varlen = kVarlen < 0 ? p.cu_q != nullptr : kVarlen != 0;
  if (!varlen) {
    if (t >= p.real_rows) return false;
    r = t / p.dql;
    pos = p.seq_lens[r] - p.dql + (t - r * p.dql);
    return true;
  }
  if (t >= p.cu_q[p.num_reqs]) return false;
  int lo = 0, hi = p.num_reqs - 1;  // the last r with cu_q[r] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu_q[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  r = lo;
  pos = p.ctx_lens[r] + (t - p.cu_q[r]);
  return true;
}

}  // namespace msa
