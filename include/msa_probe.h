/*
 * msa_probe.h -- measurement aid exported by the same library as
 * msa_sparse_decode.h, kept out of the decode ABI: nothing on the decode path
 * calls it, and a decode caller never needs it.  It exists so a benchmark can
 * time the memory traffic of the attend's own page gathers apart from the
 * attend's compute and fixed costs (the HBM roofline of the gather is the
 * bound the decode step is measured against).
 */
#ifndef MSA_PROBE_H_
#define MSA_PROBE_H_

#include <stdint.h>

#include "msa_sparse_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Memory-rate probe (a measurement aid, not part of the attend): reads byte
 * runs of a device buffer and nothing else, so that the rate of the attend's
 * own page gathers can be measured apart from its compute and fixed costs.
 *   base, buffer_bytes: the buffer (16-byte aligned, buffer_bytes >= 16).
 *   run_offsets: int64 [num_runs], byte offsets from base; run_bytes: int32
 *     [num_runs], each a multiple of 16 in 16..32768.  A run that is
 *     misaligned, out of that range or not inside the buffer is skipped
 *     (nothing read) and counted.
 *   wg_first_run: int32 [num_workgroups + 1]; workgroup w reads runs
 *     wg_first_run[w] .. wg_first_run[w+1]-1 in order (the range is clamped
 *     into [0, num_runs]; at most 512 runs per workgroup, the rest counted as
 *     skipped).
 *   out: uint32 [2 * num_workgroups]; out[2w] = XOR of every 32-bit word
 *     workgroup w read, out[2w+1] = its number of skipped runs.
 * All arrays are device memory owned by the caller; asynchronous on stream
 * (hipStream_t or NULL).  num_workgroups = 0 launches nothing. */
msa_status msa_probe_read_runs(const void* base, int64_t buffer_bytes,
                               const int64_t* run_offsets, const int32_t* run_bytes,
                               int32_t num_runs, const int32_t* wg_first_run,
                               int32_t num_workgroups, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBE_H_ */
