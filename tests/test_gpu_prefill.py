"""GPU parity of the ragged prefill attend against the float64 oracle.

Shapes: the test page's prefill test (q_lens 300/128/77 over seq_lens
300/640/1100, every causally visible page selected, bf16 q and an fp8 q with
q_scale 0.5), chunked prefill over long contexts with an empty request and
padding rows, 63 / 64 / 70 short requests, a graph replayed with new chunk boundaries, and the chunked
prefill workload at full size on sampled rows.  Tolerance as for decode.
"""
import numpy as np
import pytest
import torch

from workloads import gen

from gpu_helpers import PrefillDevCase, assert_parity, oracle_prefill, to_f64

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("heads", [(64, 4), (16, 1)])
@pytest.mark.parametrize("qfmt", [(gen.Q_BF16, 1.0), (gen.Q_FP8, 0.5)])
@pytest.mark.parametrize("splits", [0, 3])
def test_prefill_test_page_shape(heads, qfmt, splits):
    _banner(f"prefill q_lens 300/128/77 heads={heads} q={qfmt} splits={splits}")
    case = gen.make_prefill_case(41, [300, 128, 77], [300, 640, 1100], heads[0], heads[1],
                                 q_dtype=qfmt[0], q_scale=qfmt[1])
    case.k_scale, case.v_scale = 0.5, 2.0
    d = PrefillDevCase(case)
    d.run(d.plan(splits))
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_prefill(case), what="prefill test-page shape")


@pytest.mark.parametrize("tile_rows", [1, 2, 4])
@pytest.mark.parametrize("kvd", [gen.KV_FP8, gen.KV_BF16, gen.KV_E5M2])
def test_prefill_chunks_over_context_with_empty_request_and_padding(kvd, tile_rows):
    _banner(f"chunked prefill kv={kvd} tile_rows={tile_rows}")
    case = gen.make_prefill_case(42, [37, 0, 200, 1, 64], [5000, 900, 3000, 129, 64], 32, 4,
                                 kv_dtype=kvd, rule="zipf", pad_rows=5)
    d = PrefillDevCase(case)
    d.run(d.plan(tile_rows=tile_rows))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_prefill(case), what=f"chunked prefill {kvd}")
    assert np.all(got[case.real_rows:] == 0.0)


@pytest.mark.parametrize("num_prefills", [63, 64, 70])
@pytest.mark.parametrize("tile_rows", [1, 2])
def test_prefill_many_requests(num_prefills, tile_rows):
    """The row -> request binary search over many requests (63, 64, 70):
    chunks of 0..4 rows (some requests empty) over contexts of up to 600
    tokens, plus padding rows, on single-row and 2-row tiles."""
    _banner(f"prefill {num_prefills} requests tile_rows={tile_rows}")
    rng = np.random.default_rng(44 + num_prefills)
    q_lens = rng.integers(0, 5, size=num_prefills)
    seq = q_lens + rng.integers(0, 600, size=num_prefills)
    seq = np.maximum(seq, 1)
    case = gen.make_prefill_case(45 + num_prefills, q_lens.tolist(), seq.tolist(), 16, 1,
                                 rule="zipf", pad_rows=3)
    d = PrefillDevCase(case)
    d.run(d.plan(tile_rows=tile_rows))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_prefill(case), what=f"{num_prefills} prefills")
    assert np.all(got[case.real_rows:] == 0.0)


@pytest.mark.parametrize("tile_rows", [1, 2])
def test_prefill_eight_thousand_requests(tile_rows):
    """8192 requests of 0..3 new tokens over contexts of 0..120 tokens (a
    13-level row -> request search): rows sampled across the whole range, the
    first and last row of every 512th request, and the padding rows."""
    _banner(f"prefill 8192 requests tile_rows={tile_rows}")
    rng = np.random.default_rng(47)
    n = 8192
    q_lens = rng.integers(0, 4, size=n)
    seq = np.maximum(q_lens + rng.integers(0, 121, size=n), 1)
    case = gen.make_prefill_case(48, q_lens.tolist(), seq.tolist(), 16, 1, rule="zipf",
                                 pad_rows=5)
    d = PrefillDevCase(case)
    d.run(d.plan(tile_rows=tile_rows))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    cu = case.cu_seqlens_q
    rows = set(rng.choice(case.real_rows, 256, replace=False).tolist())
    for r in range(0, n, 512):
        if cu[r + 1] > cu[r]:
            rows.update((int(cu[r]), int(cu[r + 1]) - 1))
    rows = sorted(rows)
    assert_parity(got[rows], oracle_prefill(case, rows=rows), what=f"8192 prefills, {len(rows)} rows")
    assert np.all(got[case.real_rows:] == 0.0)


def test_prefill_graph_replay_with_new_chunk_boundaries():
    """One captured run replayed after cu_seqlens_q / context_lens / top-k
    change in place (the rows they describe move; the shape does not)."""
    _banner("prefill graph replay")
    a = gen.make_prefill_case(43, [100, 60, 40], [2000, 700, 400], 16, 1, rule="zipf",
                              pad_rows=8)
    # same pool and table, other chunking of the same 208 rows
    b = gen.make_prefill_case(43, [100, 60, 40], [2000, 700, 400], 16, 1, rule="zipf",
                              pad_rows=8)
    b.q_lens = np.array([20, 130, 50], dtype=np.int32)
    b.context_lens = (b.seq_lens - b.q_lens).astype(np.int32)
    b.cu_seqlens_q = np.concatenate([[0], np.cumsum(b.q_lens)]).astype(np.int32)
    rng = np.random.default_rng(9)
    b.topk = np.full_like(a.topk, -1)
    for r in range(3):
        for i in range(int(b.q_lens[r])):
            t = int(b.cu_seqlens_q[r]) + i
            last = gen.last_visible_block(int(b.context_lens[r]) + i)
            b.topk[t, 0] = gen.pad_row(gen.pick_zipf_recent(rng, last, 16), 16)
    d = PrefillDevCase(a)
    plan = d.plan()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.run(plan)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.run(plan)
    for it, c in enumerate([a, b, a]):
        d.cu.copy_(torch.from_numpy(c.cu_seqlens_q))
        d.ctx.copy_(torch.from_numpy(c.context_lens))
        d.topk.copy_(torch.from_numpy(c.topk))
        d.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(to_f64(d.out), oracle_prefill(c), what=f"replay {it}")


def test_prefill_workload_full_size_sampled_rows():
    _banner("pf1_chunked_prefill full size")
    case = gen.make_prefill_config("pf1_chunked_prefill")
    d = PrefillDevCase(case)
    d.run(d.plan())
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = sorted(set(rng.choice(case.real_rows, 24, replace=False).tolist()
                      + [0, 1023, 1024, case.real_rows - 1]))
    assert_parity(to_f64(d.out)[rows], oracle_prefill(case, rows=rows),
                  what=f"pf1 {len(rows)} sampled rows")
