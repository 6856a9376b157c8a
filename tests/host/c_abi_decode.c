/* A plain C consumer of the decode library's C ABI (include/msa_sparse_decode.h):
 * device buffers from hipMalloc, no Python and no torch.  It runs one sparse
 * decode step through msa_sparse_decode_plan / _run / _plan_destroy and
 * checks it against closed forms of the definition (the vLLM API page
 * "vllm.models.minimax_m3.common.sparse_attention", MiniMaxM3SparseImpl):
 *
 *  - every visible V row of every page holds the same vector v, so each real
 *    row's output is v * v_scale whatever the scores (the softmax weights sum
 *    to one);
 *  - padding rows, and a row whose selections are all -1, are exact zeros
 *    (TensorRT-LLM PR #17171, flash-decoding commit: zeroed padding rows);
 *  - rows past seq_len in each request's last page and a spare page hold fp8
 *    NaN codes, so a read of a non-visible row would show in the output.
 *
 * The step runs under three plans (the plan's split choice, 2 splits merged
 * inside the attend, 8 splits with the separate merge launch), and one
 * misuse (decode_query_len 33) must come back as MSA_ERR_INVALID_ARG with a
 * message.  Exit status 0 and a last line "c-abi decode ok" on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "msa_sparse_decode.h"

enum { kBatch = 2, kDql = 2, kRows = 6, kHq = 16, kHkv = 1, kTopk = 4, kStride = 8,
       kPages = 10, kRow = 256 };

static const uint8_t kFp8Nan = 0x7f;

/* e4m3fn codes of exactly representable values (sign | exponent+7 | mantissa) */
static uint8_t v_code(int d) {
  static const uint8_t codes[8] = {0x38, 0x40, 0x30, 0xb8, 0xc0, 0xb0, 0x48, 0x00};
  return codes[d % 8]; /* 1, 2, 0.5, -1, -2, -0.5, 4, 0 */
}
static double v_value(int d) {
  static const double vals[8] = {1.0, 2.0, 0.5, -1.0, -2.0, -0.5, 4.0, 0.0};
  return vals[d % 8];
}

static uint32_t lcg(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return *s >> 8;
}

static double bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

#define HIP_OK(x)                                                             \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 2;                                                               \
    }                                                                         \
  } while (0)

int main(void) {
  if (msa_abi_version() != MSA_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header says %d\n", msa_abi_version(), MSA_ABI_VERSION);
    return 1;
  }

  /* Misuse is reported before any HIP call. */
  msa_decode_shape bad;
  memset(&bad, 0, sizeof(bad));
  bad.batch = 1; bad.decode_query_len = 33; bad.page_table_stride = 1; bad.num_q_heads = 16;
  bad.num_kv_heads = 1; bad.page_size = 128; bad.head_dim = 128; bad.topk_blocks = 4;
  bad.kv_dtype = MSA_KV_FP8_E4M3; bad.q_dtype = MSA_Q_BF16;
  msa_plan none = NULL;
  if (msa_sparse_decode_plan(&bad, 0, &none) != MSA_ERR_INVALID_ARG || none != NULL ||
      strlen(msa_last_error()) == 0) {
    fprintf(stderr, "decode_query_len 33 was not rejected\n");
    return 1;
  }

  /* Host data: two requests of 300 and 700 tokens, 2 query tokens each, plus
   * 2 padding rows; pages scattered over a pool of 10 (page 9 is spare). */
  static const int32_t seq_lens[kBatch] = {300, 700};
  static const int32_t table[kBatch][kStride] = {{7, 2, 4, 0, 0, 0, 0, 0},
                                                  {1, 8, 0, 5, 3, 6, 0, 0}};
  static uint8_t kv[kPages][kHkv][128][kRow];
  static uint16_t q[kRows][kHq][128];
  int32_t topk[kRows][kHkv][kTopk];
  uint32_t seed = 12345u;
  for (int p = 0; p < kPages; ++p)
    for (int i = 0; i < 128; ++i)
      for (int d = 0; d < 128; ++d) {
        kv[p][0][i][d] = (uint8_t)((lcg(&seed) & 0x3f) | ((lcg(&seed) & 1u) << 7)); /* |k| < 2 */
        kv[p][0][i][128 + d] = v_code(d);
      }
  /* NaN past seq_len in each request's last page, and on the spare page */
  for (int r = 0; r < kBatch; ++r) {
    const int last = (seq_lens[r] - 1) / 128;
    const int used = seq_lens[r] - last * 128;
    const int page = table[r][last];
    for (int i = used; i < 128; ++i) memset(kv[page][0][i], kFp8Nan, kRow);
  }
  memset(kv[9], kFp8Nan, sizeof(kv[9]));
  for (int t = 0; t < kRows; ++t)
    for (int h = 0; h < kHq; ++h)
      for (int d = 0; d < 128; ++d) {
        const float x = ((float)(lcg(&seed) % 2001u) - 1000.0f) / 500.0f;
        uint32_t bits;
        memcpy(&bits, &x, 4);
        q[t][h][d] = (uint16_t)(bits >> 16);
      }
  /* rows 0,1: request 0 (last block 2); rows 2,3: request 1 (last block 5);
   * row 3 selects nothing; rows 4,5 are padding */
  static const int32_t sel[kRows][kTopk] = {{2, 0, 1, -1}, {1, 2, -1, -1}, {5, 3, 0, -1},
                                            {-1, -1, -1, -1}, {-1, -1, -1, -1},
                                            {-1, -1, -1, -1}};
  memcpy(topk, sel, sizeof(topk));

  void *d_kv, *d_q, *d_out, *d_table, *d_seq, *d_topk;
  HIP_OK(hipMalloc(&d_kv, sizeof(kv)));
  HIP_OK(hipMalloc(&d_q, sizeof(q)));
  HIP_OK(hipMalloc(&d_out, sizeof(q)));
  HIP_OK(hipMalloc(&d_table, sizeof(table)));
  HIP_OK(hipMalloc(&d_seq, sizeof(seq_lens)));
  HIP_OK(hipMalloc(&d_topk, sizeof(topk)));
  HIP_OK(hipMemcpy(d_kv, kv, sizeof(kv), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_q, q, sizeof(q), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_table, table, sizeof(table), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_seq, seq_lens, sizeof(seq_lens), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_topk, topk, sizeof(topk), hipMemcpyHostToDevice));

  const int64_t kv_strides[4] = {kHkv * 128 * kRow, 128 * kRow, kRow, 1};
  const int64_t topk_strides[3] = {kHkv * kTopk, kTopk, 1};
  const float v_scale = 0.5f;
  static const int32_t split_choices[3] = {0, 2, 8};
  static uint16_t out[kRows][kHq][128];
  int failures = 0;
  for (int c = 0; c < 3; ++c) {
    msa_decode_shape s;
    memset(&s, 0, sizeof(s));
    s.batch = kBatch; s.decode_query_len = kDql; s.num_token_rows = kRows;
    s.page_table_stride = kStride; s.num_q_heads = kHq; s.num_kv_heads = kHkv;
    s.page_size = 128; s.head_dim = 128; s.topk_blocks = kTopk;
    s.kv_dtype = MSA_KV_FP8_E4M3; s.num_splits = split_choices[c]; s.q_dtype = MSA_Q_BF16;
    s.tile_rows = 1;
    msa_plan plan = NULL;
    msa_status st = msa_sparse_decode_plan(&s, 0, &plan);
    if (st != MSA_OK) {
      fprintf(stderr, "plan (splits %d): %d %s\n", split_choices[c], st, msa_last_error());
      return 1;
    }
    int32_t splits = 0;
    int64_t arena = 0;
    msa_sparse_decode_plan_info(plan, &splits, &arena, NULL);
    HIP_OK(hipMemset(d_out, 0xff, sizeof(out)));  /* NaN bf16 everywhere beforehand */
    st = msa_sparse_decode_run(plan, d_q, d_kv, kv_strides, kPages, 1.0f, 1.0f, v_scale,
                               (const int32_t*)d_table, (const int32_t*)d_seq,
                               (const int32_t*)d_topk, topk_strides, d_out,
                               1.0f / sqrtf(128.0f), NULL);
    if (st != MSA_OK) {
      fprintf(stderr, "run (splits %d): %d %s\n", splits, st, msa_last_error());
      return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, d_out, sizeof(out), hipMemcpyDeviceToHost));
    double worst = 0.0;
    for (int t = 0; t < kRows; ++t)
      for (int h = 0; h < kHq; ++h)
        for (int d = 0; d < 128; ++d) {
          const double got = bf16_to_double(out[t][h][d]);
          const int real = t < 3;  /* rows 0..2 see keys; row 3 selects none */
          const double want = real ? v_value(d) * v_scale : 0.0;
          const double err = fabs(got - want);
          if (!(err <= 1e-2 * (1.0 + fabs(want))) || (!real && got != 0.0)) {
            if (failures < 5)
              fprintf(stderr, "splits %d: out[%d][%d][%d] = %g, want %g\n", splits, t, h, d,
                      got, want);
            ++failures;
          }
          if (err > worst) worst = err;
        }
    printf("splits %d (arena %lld bytes): max abs err %.3g\n", splits, (long long)arena, worst);
    if (msa_sparse_decode_plan_destroy(plan) != MSA_OK) {
      fprintf(stderr, "destroy: %s\n", msa_last_error());
      return 1;
    }
  }
  hipFree(d_kv); hipFree(d_q); hipFree(d_out); hipFree(d_table); hipFree(d_seq);
  hipFree(d_topk);
  if (failures) {
    fprintf(stderr, "%d mismatches\n", failures);
    return 1;
  }
  printf("c-abi decode ok\n");
  return 0;
}
