/*
 * msa_sparse_decode.h -- C ABI of the MI355X (gfx950) block-sparse GQA decode
 * library: MiniMax-M3-style sparse attention decode over indexer-selected
 * 128-token KV pages, plus the indexer block-max scorer and top-k selector.
 *
 * Sources of the operation (the pages this library implements):
 *  - vLLM API page "vllm.models.minimax_m3.nvidia.msa_cutlass_sparse_decode":
 *    MSACutlassDecodePlanCache.prepare / _build_plan (plan keyed by the static
 *    shape, graph-stable mutable state, argument checks), msa_cutlass_sparse_decode
 *    (fp8 query with q_scale_float; packed cache split into K = first 128,
 *    V = last 128 of the last dim; sm_scale, k/v scales), prepare_decode_metadata.
 *  - vLLM API page "vllm.models.minimax_m3.common.sparse_attention":
 *    MiniMaxM3SparseBackend (head size 128, block size 128, bf16 / fp8 e4m3 /
 *    fp8 e5m2 KV, cache shape (num_blocks, num_kv_heads, 128, 2*128) in HND
 *    order),
 *    MiniMaxM3SparseImpl (each query attends only the indexer-selected
 *    blocks), MiniMaxM3SparseTritonImpl.forward (decode call arguments).
 *  - The same sparse-attention page: MiniMaxM3SparsePrefillMetadata
 *    (cu_seqlens_q rebased to 0, context_lens of cached tokens) and the
 *    prefill call of MiniMaxM3SparseTritonImpl.forward.
 *  - vLLM test file test_minimax_m3_msa_cutlass_sparse_decode.py: _make_topk
 *    (logical block ids per (token, kv head), -1 padding, token position
 *    seq_len - query_len + local), _make_paged_layout (one block-table row
 *    per request over a shuffled pool), static-dispatch cases (decode query
 *    length 1..32).
 *  - TensorRT-LLM PR #17171 "Custom decode kernels for MinimaxM3": split-K
 *    flash decoding with fp32 partials in a persistent arena, zeroed (not
 *    NaN) output for padding rows; per-block causal max score of q.k and a
 *    strided top-k selector.
 *
 * Conventions for every entry point:
 *  - All tensor arguments are DEVICE pointers on the plan's (or the current)
 *    HIP device, owned by the caller.  The library never frees them.
 *  - Strides are in ELEMENTS of the tensor's element type.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Launches are asynchronous; no entry point synchronises the host with the
 *    device or allocates device memory except msa_sparse_decode_plan.
 *  - A negative status is returned for misuse that the host can detect; the
 *    message is then available from msa_last_error() (thread-local).  No
 *    exception crosses the ABI.  Argument checks run before any HIP call.
 *  - Data-dependent inputs are not errors: a negative top-k entry, a block
 *    that starts after the token's position, a block id at or beyond
 *    page_table_stride, or a block-table entry outside [0, num_kv_blocks)
 *    contributes nothing.  Duplicate block ids in one row are a precondition
 *    violation (result unspecified, memory-safe).
 */
#ifndef MSA_SPARSE_DECODE_H_
#define MSA_SPARSE_DECODE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 7

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,   /* bad pointer, size, stride or alignment       */
  MSA_ERR_UNSUPPORTED = -2,   /* valid but outside what the kernels implement */
  MSA_ERR_DEVICE = -3,        /* a HIP runtime call failed (no GPU, bad device) */
  MSA_ERR_OUT_OF_MEMORY = -4  /* plan arena allocation failed                  */
} msa_status;

typedef enum msa_kv_dtype {
  MSA_KV_BF16 = 0,            /* bf16 K|V entries                              */
  MSA_KV_FP8_E4M3 = 1,        /* OCP fp8 e4m3fn K|V entries, per-tensor scale  */
  MSA_KV_FP8_E5M2 = 2,        /* OCP fp8 e5m2 K|V entries, per-tensor scale    */
  MSA_KV_MXFP4 = 3            /* 4-bit head slots, see below                   */
} msa_kv_dtype;

/* MSA_KV_MXFP4: an OCP-MX analogue of the NVFP4 head-slot page of vLLM's
 * MiniMax-M3 MSA test file (_make_nvfp4_kv_cache,
 * test_nvfp4_kv_cache_views_address_head_slots).  Each page holds, per kv head
 * h, a K slot and a V slot of 8704 bytes each:
 *   bytes [0, 8192)     128 rows x 64 bytes of OCP e2m1 codes; head dim d of a
 *                       row is the low (d even) or high (d odd) nibble of
 *                       byte d/2;
 *   bytes [8192, 8704)  128 rows x 4 OCP E8M0 block-scale codes; code s of a
 *                       row scales head dims 32s..32s+31 by 2^(code-127)
 *                       (code 255 is NaN).
 * An entry's value is e2m1 * 2^(code-127) * k_scale (K) or * v_scale (V).
 * The vLLM page layout is the cache tensor uint8 [num_blocks, 2*Hkv, 128, 68]
 * (slot 2h = K of head h, slot 2h+1 = V), i.e. kv_strides (bytes)
 * {2*Hkv*8704, 2*8704, 8704, 1}: [0] page stride, [1] head stride (K slot to
 * the next head's K slot), [2] K slot -> V slot offset, [3] must be 1; [0..2]
 * positive multiples of 16, [2] >= 8704 and <= 16 MiB.
 * Where the attend and the scorer widen 4-bit entries to bf16 they read a
 * scale code as the fp32 bit pattern code << 23: code 0 then counts as 0
 * (not 2^-127, a difference below 2^-124 per element) and code 255 as +inf
 * (a non-finite result, as NaN gives).  The fp8-q MFMA and msa_mxfp4_to_bf16
 * decode every code exactly. */

typedef enum msa_q_dtype {
  MSA_Q_BF16 = 0,             /* bf16 q                                        */
  MSA_Q_FP8_E4M3 = 1          /* OCP fp8 e4m3fn q codes; value = code * q_scale
                                 (needs an fp8 or MXFP4 KV cache)              */
} msa_q_dtype;

/* Static shape of one decode step: the plan key (batch, decode query length,
 * page-table stride, q heads, kv heads, page size, top-k) of the plan cache in
 * MSACutlassDecodePlanCache.prepare, plus KV and q dtypes, padding rows and
 * split count. */
typedef struct msa_decode_shape {
  int32_t batch;              /* requests, >= 1                                  */
  int32_t decode_query_len;   /* query tokens per request, 1..32                 */
  int32_t num_token_rows;     /* rows of q/topk/out; >= batch*decode_query_len.
                                 Rows past batch*decode_query_len are padding
                                 rows and produce exact zeros. 0 = no padding.   */
  int32_t page_table_stride;  /* elements between block-table rows, >= 1         */
  int32_t num_q_heads;        /* Hq, multiple of num_kv_heads                    */
  int32_t num_kv_heads;       /* Hkv; Hq/Hkv (the GQA group) must be 1..16       */
  int32_t page_size;          /* must be 128 (one sparse block per KV page)      */
  int32_t head_dim;           /* must be 128                                     */
  int32_t topk_blocks;        /* entries per top-k row, 1..64; 0 = dense decode:
                                 every visible block, run with topk = NULL
                                 (TensorRT-LLM PR #17171, dense-decode commit)   */
  int32_t kv_dtype;           /* msa_kv_dtype                                    */
  int32_t num_splits;         /* split-K factor over a row's live blocks; 0 lets
                                 the plan choose, else 1..16                     */
  int32_t q_dtype;            /* msa_q_dtype                                     */
  int32_t tile_rows;          /* token rows per workgroup: 0 lets the plan
                                 choose; 1 = one row per workgroup (sparse only);
                                 2 or 4 = multi-row tiles that read and widen
                                 each page shared by their rows once             */
} msa_decode_shape;

/* Static shape of one ragged prefill step (the prefill call of
 * MiniMaxM3SparseTritonImpl.forward): num_prefills requests whose query
 * chunks occupy consecutive rows of q / topk / out, as cu_seqlens_q says at
 * run time. */
typedef struct msa_prefill_shape {
  int32_t num_prefills;       /* requests, >= 1                                  */
  int32_t num_token_rows;     /* rows of q/topk/out, >= 1; rows at or past
                                 cu_seqlens_q[num_prefills] are padding rows
                                 and produce exact zeros                         */
  int32_t page_table_stride;  /* elements between block-table rows, >= 1         */
  int32_t num_q_heads;        /* as in msa_decode_shape                          */
  int32_t num_kv_heads;
  int32_t page_size;          /* must be 128                                     */
  int32_t head_dim;           /* must be 128                                     */
  int32_t topk_blocks;        /* entries per top-k row, 1..64                    */
  int32_t kv_dtype;           /* msa_kv_dtype                                    */
  int32_t q_dtype;            /* msa_q_dtype                                     */
  int32_t num_splits;         /* 0 = plan's choice, else 1..16                   */
  int32_t tile_rows;          /* as in msa_decode_shape (0 = plan's choice)      */
} msa_prefill_shape;

typedef struct msa_plan_s* msa_plan;

/* Validate `shape`, choose the launch configuration and allocate the plan's
 * persistent fp32 split-K partial arena on HIP device `device` (the only
 * allocation the library makes).
 * Defined by: vLLM MSA decode page, MSACutlassDecodePlanCache.prepare and
 * _build_plan (one plan per static shape, validated up front, whose device
 * state keeps stable addresses across graph replays); TensorRT-LLM PR #17171,
 * flash-decoding commit (split-K partials in a persistent buffer arena).
 * On success *plan_out owns that arena until msa_sparse_decode_plan_destroy.
 * A plan must not be run concurrently on two streams (the arena is shared).
 * A plan that merges its splits inside the attend also keeps one int32
 * arrival counter per work unit in the arena, zeroed here (a hipMemset and a
 * device synchronisation) and left at zero by every run that completes.  A
 * run that does not complete (its stream torn down, its process or kernel
 * killed mid-way) can leave counters non-zero, after which later runs of the
 * plan would merge wrongly without an error: destroy such a plan and make a
 * new one.  Shape errors return MSA_ERR_INVALID_ARG or MSA_ERR_UNSUPPORTED
 * before any HIP call. */
msa_status msa_sparse_decode_plan(const msa_decode_shape* shape, int device,
                                  msa_plan* plan_out);

/* Free the plan and its arena (no-op on NULL).  The caller must make sure no
 * launched run that uses the plan is still executing. */
msa_status msa_sparse_decode_plan_destroy(msa_plan plan);

/* Report the plan's split factor, partial-arena size in bytes and the
 * shape it was built for (any output pointer may be NULL).  For a prefill
 * plan, shape_out->decode_query_len is 0 and batch is num_prefills. */
msa_status msa_sparse_decode_plan_info(msa_plan plan, int32_t* num_splits,
                                       int64_t* arena_bytes,
                                       msa_decode_shape* shape_out);

/* One sparse decode step (the attend).
 * Defined by: vLLM sparse-attention page, MiniMaxM3SparseImpl (each query
 * attends only its indexer-selected KV blocks) and the decode call of
 * MiniMaxM3SparseTritonImpl.forward; vLLM MSA decode page,
 * msa_cutlass_sparse_decode (packed cache split into K = first 128 and V =
 * last 128 entries, sm_scale and the q/k/v scales); vLLM test page, _make_topk
 * (logical block ids per (token, kv head), -1 padding, token position
 * seq_len - query_len + local); TensorRT-LLM PR #17171, flash-decoding commit
 * (zeroed, not NaN, padding rows).
 * For token row t = r*dql + l (request r,
 * local token l) at position pos = seq_lens[r] - dql + l, kv head h and each q
 * head j = h*G + g (G = Hq/Hkv):
 *   out[t, j, :] = softmax_k( sm_scale * q[t,j,:] . K[k,:] ) V[k,:]
 * over the keys k = b*128 + i of every selected logical block b =
 * topk[t, h, s] with b >= 0 and b*128 <= pos, i < min(128, pos - b*128 + 1),
 * read from physical page block_table[r, b].  q is the decoded q times
 * q_scale; K and V are the decoded cache entries times k_scale / v_scale.
 * Rows with no visible key, and padding rows, are written as exact zeros.
 *
 *   q            [num_token_rows, Hq, 128], contiguous: bf16, or fp8 e4m3fn
 *                codes when the plan's q_dtype is MSA_Q_FP8_E4M3.
 *   kv_cache     packed K|V entries, logical [num_kv_blocks, Hkv, 128, 256]
 *                with strides kv_strides (elements); kv_strides[3] must be 1
 *                and the other strides must be positive multiples of 16 bytes;
 *                the row stride kv_strides[2] must be >= 256 elements and
 *                below 16 MiB (MSA_ERR_UNSUPPORTED above).
 *                HND (vLLM's default) is {Hkv*128*256, 128*256, 256, 1}.
 *                An MSA_KV_MXFP4 cache is 4-bit head slots instead, with the
 *                byte strides described at msa_kv_dtype.
 *   block_table  int32 [batch, page_table_stride] physical page ids.
 *   seq_lens     int32 [batch] device copy, including the new tokens; read on
 *                the device, so runs are graph-capturable and may change
 *                between replays.
 *   topk         int32 logical [num_token_rows, Hkv, topk_blocks] with
 *                topk_strides (elements), -1 = no block.  NULL (and
 *                topk_strides ignored) for a dense plan, which attends every
 *                block b with b*128 <= pos.
 *   out          bf16 [num_token_rows, Hq, 128], contiguous.
 *   sm_scale, q_scale, k_scale must be finite and > 0 (the kernel takes each
 *   row's maximum before applying them); v_scale must be finite.  For a bf16
 *   q pass q_scale = 1 unless the q values are to be scaled.
 */
msa_status msa_sparse_decode_run(msa_plan plan, const void* q, const void* kv_cache,
                                 const int64_t kv_strides[4], int64_t num_kv_blocks,
                                 float q_scale, float k_scale, float v_scale,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* topk, const int64_t topk_strides[3],
                                 void* out, float sm_scale, void* stream);

/* The two launches of msa_sparse_decode_run, for callers that schedule or
 * time them apart.
 * Defined by: TensorRT-LLM PR #17171, flash-decoding commit (split-K over the
 * selected blocks with fp32 partials, combined by log-sum-exp, padding rows
 * zeroed).  msa_sparse_decode_run(...) is exactly
 * msa_sparse_decode_attend(...) followed by msa_sparse_decode_merge(...) on the
 * same stream.  With one split (msa_sparse_decode_plan_info), and for
 * single-row plans (tile_rows 1) with 2 to 4 splits, whose last split to
 * finish combines the partials itself, the attend writes `out` and the merge
 * launches nothing; otherwise the attend leaves fp32 split partials in the
 * plan's arena and the merge combines them by log-sum-exp into `out`
 * (TensorRT-LLM PR #17171, flash-decoding commit: split-K with fp32
 * partials, zeroed padding rows).  The merge must use the
 * same `out`, `v_scale` and stream as the attend before it, and no other run
 * of the plan may come between them. */
msa_status msa_sparse_decode_attend(msa_plan plan, const void* q, const void* kv_cache,
                                    const int64_t kv_strides[4], int64_t num_kv_blocks,
                                    float q_scale, float k_scale, float v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* topk, const int64_t topk_strides[3],
                                    void* out, float sm_scale, void* stream);
msa_status msa_sparse_decode_merge(msa_plan plan, void* out, float v_scale, void* stream);

/* A prefill plan: the same validation, split choice and arena as
 * msa_sparse_decode_plan (destroyed by msa_sparse_decode_plan_destroy).
 * Defined by: vLLM sparse-attention page, MiniMaxM3SparsePrefillMetadata and
 * the prefill call of MiniMaxM3SparseTritonImpl.forward. */
msa_status msa_sparse_prefill_plan(const msa_prefill_shape* shape, int device,
                                   msa_plan* plan_out);

/* One ragged prefill attend (vLLM sparse-attention page, prefill call of
 * MiniMaxM3SparseTritonImpl.forward): token row t with
 * cu_seqlens_q[r] <= t < cu_seqlens_q[r+1] belongs to request r and sits at
 * pos = context_lens[r] + t - cu_seqlens_q[r]; it attends exactly as a decode
 * token at pos does (see msa_sparse_decode_run).
 *   cu_seqlens_q  int32 [num_prefills + 1] device, non-decreasing, starting at
 *                 0, last entry <= num_token_rows (a request may own no row).
 *   context_lens  int32 [num_prefills] device: cached tokens before the chunk,
 *                 so the request's keys are 0 .. context_lens[r] + q_len - 1.
 *   q, kv_cache, block_table ([num_prefills, stride]), topk, out and the
 *   scales as in msa_sparse_decode_run.  Both launches (attend, merge) are
 *   made; the inputs are read on the device, so a captured run can be
 *   replayed with new chunk boundaries.
 * Out-of-contract cu_seqlens_q (decreasing, or past num_token_rows) cannot be
 * detected on the host; the kernels stay in bounds for any values whose
 * request lookup lands in [0, num_prefills). */
msa_status msa_sparse_prefill_run(msa_plan plan, const void* q, const void* kv_cache,
                                  const int64_t kv_strides[4], int64_t num_kv_blocks,
                                  float q_scale, float k_scale, float v_scale,
                                  const int32_t* block_table, const int32_t* cu_seqlens_q,
                                  const int32_t* context_lens, const int32_t* topk,
                                  const int64_t topk_strides[3], void* out, float sm_scale,
                                  void* stream);

/* Indexer step of a full decode: per-block causal max score, then top-k.
 * Defined by: TensorRT-LLM PR #17171, indexer-scorer commit (per block, the
 * causal max of q.k over the kv head's q heads and the block's visible keys,
 * one launch sized to the batch) and its selector (a top-k over a score
 * buffer of arbitrary strides); the tie rule (the lower block id first) is
 * the full-decode-step workload statement's.
 *   score[h, b, t] = max over g < G and visible keys i of block b of
 *                    q[t, h*G+g, :] . K[block_table[r,b], h, i, :]
 * (raw dot product with q = decoded q * q_scale and K = decoded entries *
 * k_scale, no softmax scale; q_scale and k_scale finite and > 0),
 * -inf for blocks b < max_blocks that start after the token's position; then
 * topk_out[t, h, :] = the topk_k blocks with the largest score > -inf, in
 * descending score order with ties to the lower block id, padded with -1.
 *   shape        batch (1..4096), decode_query_len, num_token_rows (padding rows get
 *                -inf scores and all -1 selections), heads, page_table_stride,
 *                page_size, head_dim, kv_dtype, q_dtype are used; topk_blocks
 *                and num_splits are ignored.
 *   score        float32 logical [Hkv, max_blocks, num_token_rows] with
 *                score_strides (elements): caller-owned scratch, required
 *                (NULL is MSA_ERR_INVALID_ARG).  The call takes no plan and
 *                allocates nothing, so it has no buffer of its own to fall
 *                back on; the scores stay readable after the call.
 *   max_blocks   1..16384, at least ceil(max seq_len / 128).
 *   topk_out     int32 [num_token_rows, Hkv, topk_k], contiguous; topk_k 1..64.
 *                NULL: the scores alone (one launch), for
 *                msa_sparse_decode_select_run to select from.
 */
msa_status msa_block_score_topk(const msa_decode_shape* shape, const void* q,
                                const void* kv_cache, const int64_t kv_strides[4],
                                int64_t num_kv_blocks, float q_scale, float k_scale,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_blocks, float* score,
                                const int64_t score_strides[3], int32_t* topk_out,
                                int32_t topk_k, void* stream);

/* The selector alone: topk_out[t, h, :] from score (same layout and rule as
 * msa_block_score_topk) for num_rows rows and num_kv_heads heads.
 * Defined by: TensorRT-LLM PR #17171, indexer-scorer commit (the selector
 * reads a score buffer of arbitrary strides); ties to the lower block id as
 * in the full-decode-step workload statement.  NaN and -inf scores are never
 * selected; -0 and +0 tie. */
msa_status msa_topk_select(const float* score, const int64_t score_strides[3],
                           int32_t num_kv_heads, int32_t max_blocks, int32_t num_rows,
                           int32_t* topk_out, int32_t topk_k, void* stream);

/* The selector and the attend of an indexed decode step in one launch: each
 * (token row, kv head) workgroup of a single-row plan selects its row's
 * top-k blocks from `score` (the msa_topk_select rule: the topk_blocks
 * blocks with the largest score > -inf, ties to the lower block id, -1
 * padding) and attends over them as msa_sparse_decode_run would over that
 * top-k row.  No top-k row goes through memory between the two.
 * Defined by: TensorRT-LLM PR #17171, indexer-scorer commit (block scores ->
 * top-k selector -> the sparse attend over the selected blocks) and
 * flash-decoding commit (the attend); vLLM sparse-attention page,
 * MiniMaxM3SparseImpl (the attend over the selected blocks).
 *   plan         a sparse decode plan with tile_rows 1 (single-row); a dense,
 *                prefill or multi-row plan is MSA_ERR_UNSUPPORTED.  Splits as
 *                for msa_sparse_decode_run (each split selects the same row).
 *   q .. seq_lens, out, sm_scale, stream: as for msa_sparse_decode_run.
 *   score        float32 logical [Hkv, max_blocks, num_token_rows] with
 *                score_strides (elements), e.g. msa_block_score_topk's buffer;
 *                read only.
 *   max_blocks   1..16384.  Up to 2048 blocks the selecting workgroup keeps
 *                two wavefronts per SIMD; larger rows run at one.
 *   topk_out     NULL, or int32 [num_token_rows, Hkv, topk_blocks],
 *                contiguous: receives the selection (padding rows all -1),
 *                exactly what msa_topk_select gives for the same scores.
 */
msa_status msa_sparse_decode_select_run(msa_plan plan, const void* q, const void* kv_cache,
                                        const int64_t kv_strides[4], int64_t num_kv_blocks,
                                        float q_scale, float k_scale, float v_scale,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        const float* score, const int64_t score_strides[3],
                                        int32_t max_blocks, int32_t* topk_out, void* out,
                                        float sm_scale, void* stream);

/* Decode n OCP fp8 e4m3fn codes to bf16 with the same in-register conversion
 * the attend uses (a self-check of the conversion path).  The format is the
 * vLLM test page's torch.float8_e4m3fn cache.  in: uint8[n],
 * out: bf16 bits uint16[n], device pointers, n >= 1. */
msa_status msa_fp8_e4m3_to_bf16(const void* in, void* out, int64_t n, void* stream);
/* The same for OCP fp8 e5m2 codes (the vLLM sparse-attention page lists an
 * fp8_e5m2 KV cache among the backend's cache dtypes). */
msa_status msa_fp8_e5m2_to_bf16(const void* in, void* out, int64_t n, void* stream);

/* Dequantize an MSA_KV_MXFP4 cache (layout and kv_strides as described at
 * msa_kv_dtype) to packed bf16 K|V rows, with the block scales applied and
 * the global k/v scales not: out is bf16 bits, contiguous
 * [num_kv_blocks, num_kv_heads, 128, 256] (K = entries 0..127, V = 128..255),
 * computed with the attend's own in-register conversion.  The result is exact
 * (e2m1 times a power of two is a bf16 value).  The vLLM test file's NVFP4
 * tests compare the MSA kernels against a Triton path run on such a
 * dequantized cache. */
msa_status msa_mxfp4_to_bf16(const void* kv_cache, const int64_t kv_strides[4],
                             int64_t num_kv_blocks, int32_t num_kv_heads, void* out,
                             void* stream);

/* Bytes of the static device scratch msa_sparse_decode_run_noalloc uses. */
#define MSA_NOALLOC_SCRATCH_BYTES (64LL << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * decode step as msa_sparse_decode_run (same arguments, same result) without a
 * plan: `shape` and `device` are what msa_sparse_decode_plan would take, and
 * the launch is configured the same way on the host, except that several
 * splits are always merged by a separate merge launch.  The fp32 split
 * partials go to a static device array of MSA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds on every device it runs on until the process ends;
 * the call allocates nothing and frees nothing.  A shape whose partials need
 * more (num_token_rows * num_q_heads * splits * 520 bytes when splits > 1)
 * returns MSA_ERR_UNSUPPORTED with a message; pass fewer num_splits, or use a
 * plan.  Every call on one device shares that device's array, so calls that
 * overlap on one GPU (two streams or two host threads) race and give wrong
 * results: serialize them.  The first call on each device looks up the
 * array's address there (hipGetSymbolAddress, a runtime query, no
 * allocation); make it outside graph capture.  Errors as for
 * msa_sparse_decode_plan and msa_sparse_decode_run. */
msa_status msa_sparse_decode_run_noalloc(const msa_decode_shape* shape, int device,
                                         const void* q, const void* kv_cache,
                                         const int64_t kv_strides[4], int64_t num_kv_blocks,
                                         float q_scale, float k_scale, float v_scale,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         const int32_t* topk, const int64_t topk_strides[3],
                                         void* out, float sm_scale, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* msa_last_error(void);

/* MSA_ABI_VERSION of the built library. */
int32_t msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_SPARSE_DECODE_H_ */
