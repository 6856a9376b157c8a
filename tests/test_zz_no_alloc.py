"""The no-allocation decode entry point against the plan-based one.

msa_sparse_decode_run_noalloc runs the decode step with the split partials in
the library's static per-device scratch instead of a plan's arena.  Two calls
in a row, the second on a smaller input (so the first call's partials are
still in the scratch when the second runs), each compared with
msa_sparse_decode_run on the same inputs to the parity bar, and with the
float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_gqa_decode_amd as msa
from workloads import gen

from gpu_helpers import DevCase, assert_parity, oracle_attend, to_f64

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _noalloc(d: DevCase, splits: int, tile_rows: int):
    c = d.case
    out = d.new_out()
    msa.msa_sparse_decode_run_noalloc(
        d.q, d.kv, d.block_table, d.seq_lens, d.topk, out, decode_query_len=c.dql,
        num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, topk_blocks=c.topk_k,
        kv_dtype=d.kv_dtype, q_dtype=d.q_dtype, num_token_rows=c.num_token_rows,
        num_splits=splits, tile_rows=tile_rows, sm_scale=c.sm_scale, k_scale=c.k_scale,
        v_scale=c.v_scale, q_scale=c.q_scale)
    return out


def test_noalloc_matches_plan_run_twice_in_a_row():
    big = gen.make_random_case(601, 8, 4, 64, 4, 16, 2000, 40000, pad_rows=3)
    small = gen.make_random_case(602, 3, 2, 16, 1, 8, 500, 9000, pad_rows=1)
    for case, splits, tile_rows in ((big, 8, 1), (small, 3, 1)):
        _banner(f"no-alloc decode: rows {case.num_token_rows}, heads "
                f"({case.num_q_heads},{case.num_kv_heads}), splits {splits}, "
                f"tile_rows {tile_rows}")
        d = DevCase(case)
        got = _noalloc(d, splits, tile_rows)
        ref = d.run(d.plan(splits, tile_rows=tile_rows), out=d.new_out())
        torch.cuda.synchronize()
        assert_parity(to_f64(got), to_f64(ref), what="no-alloc vs plan run")
        assert_parity(to_f64(got), oracle_attend(case), what="no-alloc vs oracle")
        pad = slice(case.batch * case.dql, case.num_token_rows)
        assert torch.all(got[pad].float() == 0)
