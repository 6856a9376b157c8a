"""GPU parity of the multi-row tile kernels and of dense decode.

The tile kernels (several token rows per workgroup, each page shared by its
rows read once: pages staged in registers for 2- and 4-row tiles, through an
LDS ring for 8-row tiles over 8-bit caches) must give
what the oracle gives for any tile size: the randomized decode cases and the
format cases are rerun on 2-, 4- and 8-row tiles,
the single-row kernel is checked on a long decode query length, a graph of
sparse tiles is replayed with the requests' length order reversed, and dense
decode (every visible block, no top-k) is checked on the test page's shapes,
randomized shapes (query lengths 1..8, padding rows, NHD, every split count,
all formats), a graph replayed with new lengths and the TP1-shaped dense
workload at full size on sampled rows.  Tolerance as for decode.
"""
import numpy as np
import pytest
import torch

from workloads import gen

import block_sparse_gqa_decode_amd as msa
from gpu_helpers import DevCase, assert_parity, oracle_attend, oracle_dense, to_f64

import test_gpu_parity as base

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("tile_rows", [2, 4, 8])
@pytest.mark.parametrize("seed,batch,dql,hq,hkv,k,lo,hi,kvd,pad,neg,splits,layout",
                         base.RANDOM_CASES)
def test_random_cases_on_tiles(tile_rows, seed, batch, dql, hq, hkv, k, lo, hi, kvd, pad, neg,
                               splits, layout):
    _banner(f"tiles={tile_rows} random seed={seed} dql={dql} heads=({hq},{hkv}) k={k} "
            f"splits={splits} layout={layout}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, k, lo, hi, kv_dtype=kvd,
                                pad_rows=pad, neg_frac=neg)
    d = DevCase(case, layout=layout)
    if tile_rows == 8 and kvd == gen.KV_BF16:
        with pytest.raises(msa.MsaUnsupported, match="8-row tiles"):
            d.plan(splits, tile_rows=tile_rows)
        return
    plan = d.plan(splits, tile_rows=tile_rows)
    assert plan.tile_rows == tile_rows
    d.run(plan)
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_attend(case), what=f"tiles random {seed}")
    assert np.all(got[case.real_rows:] == 0.0)


@pytest.mark.parametrize("tile_rows", [2, 4, 8])
@pytest.mark.parametrize("seed,batch,dql,hq,hkv,k,lo,hi,kvd,qd,qs,pad,neg,splits,layout",
                         base.FORMAT_RANDOM_CASES)
def test_format_cases_on_tiles(tile_rows, seed, batch, dql, hq, hkv, k, lo, hi, kvd, qd, qs,
                               pad, neg, splits, layout):
    _banner(f"tiles={tile_rows} random seed={seed} kv={kvd} q={qd}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, k, lo, hi, kv_dtype=kvd,
                                pad_rows=pad, neg_frac=neg, q_dtype=qd, q_scale=qs)
    case.k_scale, case.v_scale = 0.5, 1.5
    d = DevCase(case, layout=layout)
    d.run(d.plan(splits, tile_rows=tile_rows))
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case), what=f"tiles format {seed}")


@pytest.mark.parametrize("tile_rows", [2, 4])
def test_tiles_graph_replay_with_the_length_order_reversed(tile_rows):
    """Sparse 2- and 4-row tiles deal the requests longest first, ranking them
    by seq_lens on the device at every launch.  A graph captured with one
    length order is replayed with the order reversed, then restored, with
    fresh top-k rows for each; every replay is checked against the oracle."""
    _banner(f"tiles={tile_rows} graph replay, request length order reversed")
    B, dql = 8, 4
    # tables and pages for 6000 tokens per request; shorter lengths use a prefix
    case = gen.make_random_case(192, B, dql, 64, 4, 16, 6000, 6000, pad_rows=2)
    rng = np.random.default_rng(193)
    lens = np.array([6000, 5000, 4100, 3500, 600, 420, 250, 130], dtype=np.int32)
    orders = [lens, lens[::-1].copy(), lens]

    def topk_for(seq):
        return gen._topk_rows(rng, seq, dql, case.num_kv_heads, 16,
                              lambda r, last: gen.pick_uniform(rng, last, 16), True,
                              pad_rows=2)

    d = DevCase(case)
    plan = d.plan(tile_rows=tile_rows)
    assert plan.tile_rows == tile_rows
    d.seq_lens.copy_(torch.from_numpy(orders[0]))
    d.topk.copy_(torch.from_numpy(topk_for(orders[0])))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run(plan)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(plan)
    for it, seq in enumerate(orders):
        tk = topk_for(seq)
        d.seq_lens.copy_(torch.from_numpy(seq))
        d.topk.copy_(torch.from_numpy(tk))
        d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        case.seq_lens, case.topk = seq, tk
        got = to_f64(d.out)
        assert_parity(got, oracle_attend(case), what=f"replay {it}, lengths {seq.tolist()}")
        assert np.all(got[case.real_rows:] == 0.0)


def test_long_query_length_single_row_and_tiles_agree_with_oracle():
    _banner("dql=32, single-row kernel vs 2-, 4- and 8-row tiles")
    case = gen.make_random_case(171, 3, 32, 64, 4, 16, 300, 20000, pad_rows=3)
    d = DevCase(case)
    ref = oracle_attend(case)
    for tr in (1, 2, 4, 8):
        d.out.fill_(float("nan"))
        plan = d.plan(tile_rows=tr)
        assert plan.tile_rows == tr
        d.run(plan)
        torch.cuda.synchronize()
        assert_parity(to_f64(d.out), ref, what=f"dql=32 tile_rows={tr}")


# ---------------------------------------------------------------------------
# dense decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hq,hkv,pairs,dql", [(64, 4, 8, 1), (64, 4, 8, 4), (16, 1, 16, 4),
                                              (64, 4, 8, 8)])
def test_dense_decode_test_page_shapes(hq, hkv, pairs, dql):
    _banner(f"dense p3 heads=({hq},{hkv}) pairs={pairs} dql={dql}")
    case = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=(257, 513), seed=0)
    d = DevCase(case)
    plan = d.plan(dense=True)
    assert plan.dense
    d.run(plan)
    torch.cuda.synchronize()
    # every visible page selected is the same computation as dense
    assert_parity(to_f64(d.out), oracle_attend(case), what="dense p3")


DENSE_CASES = [
    # seed, batch, dql, hq, hkv, lo, hi, kv, q, q_scale, pad, splits, tile_rows, layout
    (181, 4, 1, 64, 4, 1, 9000, gen.KV_FP8, gen.Q_BF16, 1.0, 0, 0, 0, "hnd"),
    (182, 3, 4, 16, 1, 2000, 30000, gen.KV_FP8, gen.Q_FP8, 0.5, 2, 0, 0, "hnd"),
    (183, 2, 8, 64, 4, 100, 5000, gen.KV_BF16, gen.Q_BF16, 1.0, 1, 3, 4, "nhd"),
    (184, 5, 3, 32, 4, 1, 3000, gen.KV_E5M2, gen.Q_BF16, 1.0, 0, 16, 4, "hnd"),
    (185, 2, 5, 16, 2, 5, 700, gen.KV_E5M2, gen.Q_FP8, 2.0, 3, 1, 2, "nhd"),
    (186, 2, 2, 12, 3, 40000, 60000, gen.KV_FP8, gen.Q_BF16, 1.0, 0, 0, 4, "hnd"),
    (188, 3, 8, 64, 4, 1, 9000, gen.KV_FP8, gen.Q_BF16, 1.0, 2, 0, 8, "hnd"),
    (189, 2, 11, 16, 1, 300, 4000, gen.KV_E5M2, gen.Q_FP8, 0.5, 1, 5, 8, "nhd"),
    # seq_len below dql: the first rows of such a request see no key (exact zeros)
    (190, 4, 4, 16, 1, 1, 6, gen.KV_FP8, gen.Q_BF16, 1.0, 1, 0, 2, "hnd"),
    (191, 3, 8, 64, 4, 1, 10, gen.KV_FP8, gen.Q_FP8, 0.5, 0, 2, 4, "nhd"),
]


@pytest.mark.parametrize("seed,batch,dql,hq,hkv,lo,hi,kvd,qd,qs,pad,splits,tile_rows,layout",
                         DENSE_CASES)
def test_dense_decode_random(seed, batch, dql, hq, hkv, lo, hi, kvd, qd, qs, pad, splits,
                             tile_rows, layout):
    _banner(f"dense seed={seed} B={batch} dql={dql} heads=({hq},{hkv}) seq=[{lo},{hi}] "
            f"kv={kvd} q={qd} splits={splits} tiles={tile_rows} layout={layout}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, 4, lo, hi, kv_dtype=kvd,
                                pad_rows=pad, q_dtype=qd, q_scale=qs)
    case.k_scale, case.v_scale = 0.75, 1.25
    d = DevCase(case, layout=layout)
    d.run(d.plan(splits, tile_rows=tile_rows, dense=True))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_dense(case), what=f"dense {seed}")
    assert np.all(got[case.real_rows:] == 0.0)


def test_dense_decode_graph_replay_with_new_lengths():
    _banner("dense graph replay")
    case = gen.make_random_case(187, 4, 4, 64, 4, 4, 3000, 9000)
    d = DevCase(case)
    plan = d.plan(dense=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run(plan)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(plan)
    for it, lens in enumerate([case.seq_lens, np.minimum(case.seq_lens, 700) - 3,
                               case.seq_lens]):
        c = gen.make_random_case(187, 4, 4, 64, 4, 4, 3000, 9000)
        c.seq_lens = np.asarray(lens, dtype=np.int32)
        d.seq_lens.copy_(torch.from_numpy(c.seq_lens))
        d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(to_f64(d.out), oracle_dense(c), what=f"dense replay {it}")


def test_dense_workload_full_size_sampled_rows():
    _banner("d1_dense_tp1 full size")
    case = gen.make_dense_config("d1_dense_tp1")
    d = DevCase(case)
    plan = d.plan(dense=True)
    d.run(plan)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    rows = sorted(set(rng.choice(case.real_rows, 6, replace=False).tolist()
                      + [int(np.argmax(case.seq_lens)) * case.dql + 3]))
    assert_parity(to_f64(d.out)[rows], oracle_dense(case, rows=rows),
                  what=f"dense full size {len(rows)} rows (splits {plan.num_splits})")
