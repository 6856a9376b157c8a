"""GPU parity of the HIP decode path against the float64 oracle.

Every case is seeded and synthetic (workloads/gen.py).  Shapes follow the
pages: the test page's parity shapes (seq_lens 257/513 then 129/385 with the
same plan, then a graph replay; heads (64,4) and (16,1); query lengths
1,2,3,4,8), the five named workloads at full size on sampled rows, and
randomized edge cases (-1 padding, padding rows, G < 16, NHD strides,
transposed top-k views, non-unit scales, every split count), and the other
input formats: fp8 e5m2 KV and fp8 e4m3 q with a q scale.
Tolerance: max abs <= 1e-2, relative L2 <= 1e-2, elementwise
|a-o| <= 1e-2 + 1e-2|o| on the bf16 outputs.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_decode_amd as msa
from oracle import msa_oracle as om
from workloads import gen

from gpu_helpers import DevCase, assert_parity, oracle_attend, oracle_dense, oracle_scores, to_f64

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# the fp8 conversion the attend uses
# ---------------------------------------------------------------------------

def test_fp8_conversion_exhaustive():
    _banner("fp8 e4m3fn -> bf16, all 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(5).cuda()
    out = torch.empty(codes.numel(), dtype=torch.bfloat16, device="cuda")
    msa.msa_fp8_e4m3_to_bf16(codes, out)
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = np.tile(om.decode_e4m3fn(np.arange(256)), 5)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_fp8_e5m2_conversion_exhaustive():
    _banner("fp8 e5m2 -> bf16, all 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(5).cuda()
    out = torch.empty(codes.numel(), dtype=torch.bfloat16, device="cuda")
    msa.msa_fp8_e5m2_to_bf16(codes, out)
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = np.tile(om.decode_e5m2(np.arange(256)), 5)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])            # +-inf included


# ---------------------------------------------------------------------------
# the test page's shapes
# ---------------------------------------------------------------------------

P3_CASES = [
    (64, 4, 8, 1, True), (64, 4, 8, 2, False), (64, 4, 8, 3, False), (64, 4, 8, 4, True),
    (64, 4, 8, 8, False), (16, 1, 8, 1, True), (16, 1, 16, 4, True),
]


@pytest.mark.parametrize("hq,hkv,pairs,dql,capture", P3_CASES)
def test_p3_shapes_with_replanned_lengths_and_graph(hq, hkv, pairs, dql, capture):
    _banner(f"p3 heads=({hq},{hkv}) pairs={pairs} dql={dql} capture={capture}")
    case = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=(257, 513), seed=0)
    d = DevCase(case)
    plan = d.plan()
    d.run(plan)
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case), what="seq 257/513")

    # Same plan, ragged lengths changed in place (129/385).
    case2 = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=(257, 513), seed=0)
    case2.seq_lens = np.array([129, 385] * pairs, dtype=np.int32)
    case2.topk = gen.every_visible_topk(case2.seq_lens, hkv, dql, 16)
    d.seq_lens.copy_(torch.from_numpy(case2.seq_lens))
    d.topk.copy_(torch.from_numpy(case2.topk))
    d.run(plan)
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case2), what="seq 129/385, same plan")

    if capture:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            d.run(plan)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            d.run(plan)
        for it, (pattern, c) in enumerate([((257, 513), case), ((129, 385), case2),
                                           ((257, 513), case)]):
            d.seq_lens.copy_(torch.from_numpy(c.seq_lens))
            d.topk.copy_(torch.from_numpy(c.topk))
            d.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_parity(to_f64(d.out), oracle_attend(c), what=f"graph replay {it} {pattern}")


# (kv format, q format, q scale): the test page runs the fp8-q interface with
# q_scale 1.0; e5m2 is the backend's other fp8 cache format.
FORMATS = [(gen.KV_FP8, gen.Q_FP8, 1.0), (gen.KV_E5M2, gen.Q_BF16, 1.0),
           (gen.KV_E5M2, gen.Q_FP8, 0.5)]


@pytest.mark.parametrize("hq,hkv,pairs,dql", [(64, 4, 8, 4), (16, 1, 16, 4), (64, 4, 8, 1)])
@pytest.mark.parametrize("fmt", FORMATS)
def test_p3_shapes_other_formats(hq, hkv, pairs, dql, fmt):
    kvd, qd, qs = fmt
    _banner(f"p3 heads=({hq},{hkv}) pairs={pairs} dql={dql} kv={kvd} q={qd} q_scale={qs}")
    case = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=(257, 513), seed=0,
                            kv_dtype=kvd, q_dtype=qd, q_scale=qs)
    d = DevCase(case)
    d.run(d.plan())
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case), what=f"p3 {kvd}/{qd}")


# ---------------------------------------------------------------------------
# the tiny bf16 workload and randomized edge cases
# ---------------------------------------------------------------------------

def test_c1_tiny_bf16_all_rows():
    _banner("c1 tiny bf16")
    case = gen.make_config("c1_tiny_bf16")
    d = DevCase(case)
    for splits in (0, 1, 2, 4):
        d.out.fill_(float("nan"))
        d.run(d.plan(splits))
        torch.cuda.synchronize()
        assert_parity(to_f64(d.out), oracle_attend(case), what=f"c1 splits={splits}")


RANDOM_CASES = [
    # seed, batch, dql, hq, hkv, k, seq_lo, seq_hi, kv_dtype, pad, neg_frac, splits, layout
    (101, 3, 1, 16, 1, 16, 1, 3000, gen.KV_FP8, 0, 0.0, 0, "hnd"),
    (102, 4, 4, 64, 4, 16, 300, 5000, gen.KV_FP8, 2, 0.2, 0, "hnd"),
    (103, 2, 8, 32, 4, 8, 129, 1200, gen.KV_BF16, 1, 0.1, 3, "hnd"),
    (104, 5, 2, 16, 4, 12, 1, 2500, gen.KV_FP8, 3, 0.3, 16, "hnd"),
    (105, 3, 3, 8, 8, 5, 100, 700, gen.KV_FP8, 0, 0.0, 1, "nhd"),
    (106, 2, 32, 64, 4, 16, 200, 1900, gen.KV_FP8, 4, 0.0, 0, "hnd"),
    (107, 6, 1, 12, 3, 64, 5000, 9000, gen.KV_FP8, 0, 0.5, 2, "nhd"),
    (108, 2, 5, 16, 1, 16, 1, 40, gen.KV_BF16, 2, 0.0, 8, "hnd"),
    # top-1 (the causal last block only); forced to 2 splits every unit has
    # an empty split, which the in-kernel merge must weigh as zero
    (109, 4, 2, 16, 2, 1, 1, 3000, gen.KV_FP8, 1, 0.0, 0, "hnd"),
    (110, 4, 2, 16, 2, 1, 1, 3000, gen.KV_FP8, 1, 0.0, 2, "hnd"),
]


@pytest.mark.parametrize("seed,batch,dql,hq,hkv,k,lo,hi,kvd,pad,neg,splits,layout",
                         RANDOM_CASES)
def test_random_cases(seed, batch, dql, hq, hkv, k, lo, hi, kvd, pad, neg, splits, layout):
    _banner(f"random seed={seed} B={batch} dql={dql} heads=({hq},{hkv}) k={k} "
            f"kv={kvd} pad={pad} splits={splits} layout={layout}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, k, lo, hi, kv_dtype=kvd,
                                pad_rows=pad, neg_frac=neg)
    d = DevCase(case, layout=layout)
    d.run(d.plan(splits))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    ref = oracle_attend(case)
    assert_parity(got, ref, what=f"random {seed}")
    assert np.all(got[case.real_rows:] == 0.0)


def test_scales_and_transposed_topk_view():
    _banner("k/v scales + head-major top-k view")
    case = gen.make_random_case(111, 4, 4, 64, 4, 16, 400, 4000)
    case.k_scale, case.v_scale = 0.5, 1.75
    d = DevCase(case)
    # Head-major physical buffer [Hkv, rows, k] viewed as [rows, Hkv, k].
    tk_hm = torch.from_numpy(np.ascontiguousarray(case.topk.transpose(1, 0, 2))).cuda()
    d.run(d.plan(), topk=tk_hm.transpose(0, 1))
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case), what="scales + strided topk")


def test_all_minus_one_and_padding_rows_are_exact_zeros():
    _banner("zero rows")
    case = gen.make_random_case(112, 4, 2, 16, 1, 16, 500, 3000, pad_rows=3)
    topk = case.topk.copy()
    topk[1] = -1
    topk[4, 0, :] = -1
    case.topk = topk
    d = DevCase(case)
    for splits in (1, 4):
        d.out.fill_(float("nan"))
        d.run(d.plan(splits))
        torch.cuda.synchronize()
        got = to_f64(d.out)
        for t in (1, 4, 8, 9, 10):
            assert np.all(got[t] == 0.0) and not np.signbit(got[t]).any(), (t, splits)
        assert_parity(got, oracle_attend(case), what=f"zero rows splits={splits}")


def test_invisible_indices_and_out_of_range_blocks_are_skipped():
    _banner("invisible / beyond-table indices")
    case = gen.make_random_case(113, 3, 4, 16, 1, 16, 600, 2000, stride_extra=0)
    topk = case.topk.copy()
    rng = np.random.default_rng(0)
    for t in range(case.real_rows):
        r, loc = divmod(t, case.dql)
        pos = int(case.seq_lens[r]) - case.dql + loc
        slots = rng.choice(16, size=2, replace=False)
        topk[t, 0, slots[0]] = pos // 128 + 1             # starts after the position
        topk[t, 0, slots[1]] = case.block_table.shape[1] + 7  # beyond the table row
    case_ref = gen.make_random_case(113, 3, 4, 16, 1, 16, 600, 2000)
    case_ref.topk = topk
    d = DevCase(case)
    d.run(d.plan(), topk=torch.from_numpy(topk).cuda())
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_attend(case_ref), what="skipped indices")


def test_out_of_pool_table_entries_are_skipped():
    """Block-table entries that name no page of the pool (-1, num_blocks,
    num_blocks + 1000) for about a third of each request's used blocks: the
    attend skips those blocks (single-row with and without the in-kernel
    merge, 2-row tiles, dense decode on 4-row tiles) and the scorer leaves
    them at -inf, as the oracle does on the same table."""
    _banner("out-of-pool block-table entries")
    case = gen.make_random_case(114, 3, 4, 32, 2, 12, 300, 3000, pad_rows=2)
    rng = np.random.default_rng(9)
    nb = case.kv.shape[0]
    bt = case.block_table.copy()
    for r, s in enumerate(case.seq_lens):
        used = gen.pages_for(int(s))
        for b in rng.choice(used, size=max(1, used // 3), replace=False):
            bt[r, b] = rng.choice([-1, nb, nb + 1000])
    case.block_table = bt
    d = DevCase(case)
    ref = oracle_attend(case)
    for splits, tile_rows in ((1, 1), (2, 1), (8, 1), (0, 2)):
        d.out.fill_(float("nan"))
        d.run(d.plan(splits, tile_rows=tile_rows))
        torch.cuda.synchronize()
        assert_parity(to_f64(d.out), ref, what=f"out-of-pool splits={splits} tiles={tile_rows}")
    d.out.fill_(float("nan"))
    d.run(d.plan(0, tile_rows=4, dense=True))
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_dense(case), what="out-of-pool dense")
    mb = case.max_blocks
    score, _ = _run_scorer(d, mb, 12)
    _scores_close(score[:, :, :case.real_rows], oracle_scores(case, mb), case)


FORMAT_RANDOM_CASES = [
    # seed, batch, dql, hq, hkv, k, seq_lo, seq_hi, kv, q, q_scale, pad, neg, splits, layout
    (161, 4, 4, 64, 4, 16, 300, 5000, gen.KV_FP8, gen.Q_FP8, 0.5, 2, 0.2, 0, "hnd"),
    (162, 3, 2, 16, 4, 12, 1, 2500, gen.KV_E5M2, gen.Q_BF16, 1.0, 3, 0.3, 4, "nhd"),
    (163, 2, 8, 32, 4, 8, 129, 1200, gen.KV_E5M2, gen.Q_FP8, 0.25, 1, 0.1, 3, "hnd"),
    (164, 5, 1, 12, 3, 64, 5000, 9000, gen.KV_FP8, gen.Q_FP8, 2.0, 0, 0.5, 16, "nhd"),
]


@pytest.mark.parametrize("seed,batch,dql,hq,hkv,k,lo,hi,kvd,qd,qs,pad,neg,splits,layout",
                         FORMAT_RANDOM_CASES)
def test_random_cases_other_formats(seed, batch, dql, hq, hkv, k, lo, hi, kvd, qd, qs, pad,
                                    neg, splits, layout):
    _banner(f"random seed={seed} B={batch} dql={dql} heads=({hq},{hkv}) k={k} kv={kvd} "
            f"q={qd} q_scale={qs} pad={pad} splits={splits} layout={layout}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, k, lo, hi, kv_dtype=kvd,
                                pad_rows=pad, neg_frac=neg, q_dtype=qd, q_scale=qs)
    case.k_scale, case.v_scale = 0.5, 1.5
    d = DevCase(case, layout=layout)
    d.run(d.plan(splits))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_attend(case), what=f"random {seed}")
    assert np.all(got[case.real_rows:] == 0.0)


def test_deterministic_bitwise():
    _banner("determinism")
    case = gen.make_random_case(114, 8, 4, 16, 1, 16, 2000, 20000)
    d = DevCase(case)
    plan = d.plan()
    a = d.run(plan, out=d.new_out()).clone()
    b = d.run(plan, out=d.new_out()).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# the named workloads at full size, in the launch configuration the bench
# uses, checked on sampled rows the oracle evaluates one by one
# ---------------------------------------------------------------------------

def _sample_rows(case, n, seed):
    rng = np.random.default_rng(seed)
    rows = rng.choice(case.real_rows, size=min(n, case.real_rows), replace=False)
    extra = list(range(case.real_rows, case.num_token_rows))
    return sorted(set(rows.tolist())) + extra


@pytest.mark.parametrize("name,nrows", [("c2_tp4_fp8", 40), ("c3_tp1_fp8", 24),
                                        ("c4_spec_ragged", 48), ("c2_tp4_fp8q", 40),
                                        ("c2_tp4_e5m2", 40), ("c2_tp4_mxfp4", 40),
                                        ("c2_tp4_mxfp4_fp8q", 40)])
def test_named_workload_full_size(name, nrows):
    _banner(f"{name} full size")
    case = gen.make_config(name)
    d = DevCase(case)
    d.run(d.plan())
    torch.cuda.synchronize()
    rows = _sample_rows(case, nrows, 7)
    if name == "c4_spec_ragged":
        # make sure both long and short requests are covered
        long_rows = [t for t in range(case.real_rows)
                     if case.seq_lens[t // case.dql] == 131072][:8]
        short_rows = [t for t in range(case.real_rows)
                      if case.seq_lens[t // case.dql] < 2000][:8]
        rows = sorted(set(rows) | set(long_rows) | set(short_rows))
    got = to_f64(d.out)[rows]
    ref = oracle_attend(case, rows=rows)
    assert_parity(got, ref, what=f"{name} {len(rows)} sampled rows")
    if case.num_token_rows > case.real_rows:
        assert np.all(to_f64(d.out)[case.real_rows:] == 0.0)


# ---------------------------------------------------------------------------
# indexer scorer and top-k selector
# ---------------------------------------------------------------------------

def _run_scorer(d: DevCase, max_blocks, k, transposed=False):
    c = d.case
    rows = c.num_token_rows
    if transposed:
        # physical [Hkv, rows, blocks], logical [Hkv, blocks, rows]
        phys = torch.full((c.num_kv_heads, rows, max_blocks), float("nan"), device="cuda")
        score = phys.transpose(1, 2)
    else:
        score = torch.full((c.num_kv_heads, max_blocks, rows), float("nan"), device="cuda")
    topk_out = torch.full((rows, c.num_kv_heads, k), -7, dtype=torch.int32, device="cuda")
    d.score(score, topk_out, max_blocks, num_token_rows=rows)
    torch.cuda.synchronize()
    return score.cpu().numpy().astype(np.float64), topk_out.cpu().numpy()


def _fp8_score_tol(case):
    """Error bound for scores from the fp8 x fp8 MFMA.  That instruction sums
    its 128 products in a reduced-precision aligned accumulator: over 400 random
    16x16x128 tiles (normal, wide-dynamic-range, one-dominant-term and
    cancelling inputs) its worst error was 2^-11.3 of the largest product
    magnitude.  The bound 2^-9 * max|q| * max|k| (scales included) leaves ~5x
    headroom; a wrong index, sign or scale moves scores by O(1)."""
    qv = om.decode_query(case.q, case.q_dtype, case.q_scale)
    if case.kv_dtype == gen.KV_MXFP4:
        # |K| <= 6 * the largest finite K block scale present (4-bit products
        # meet the same accumulator)
        slots = case.kv.reshape(case.kv.shape[0], -1, 2, om.MXFP4_SLOT_BYTES)[:, :, 0]
        sc = om.decode_e8m0(np.unique(slots[..., om.MXFP4_DATA_BYTES:]))
        kmax = 6.0 * float(np.max(sc[np.isfinite(sc)])) * case.k_scale
        return 2.0 ** -9 * float(np.max(np.abs(qv))) * kmax
    present = np.zeros(256, dtype=bool)
    present[np.unique(case.kv[..., :128])] = True
    kvals = om.dequant(np.nonzero(present)[0].astype(np.uint8), case.kv_dtype, case.k_scale)
    kmax = float(np.max(np.abs(kvals[np.isfinite(kvals)])))
    return 2.0 ** -9 * float(np.max(np.abs(qv))) * kmax


def _scores_close(got, ref, case=None):
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all()
    if case is not None and case.q_dtype == gen.Q_FP8:
        tol = _fp8_score_tol(case)
    else:
        # bf16 MFMA: exact products, fp32 accumulation over 128 terms
        tol = 2e-5 * np.max(np.abs(ref[fin])) + 1e-5
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    print(f"[parity] scores: max_abs={err:.3e} tol={tol:.3e}", flush=True)
    assert err <= tol
    return tol


@pytest.mark.parametrize("kvd,dql,hq,hkv,transposed,qd,qs", [
    (gen.KV_FP8, 1, 64, 4, False, gen.Q_BF16, 1.0), (gen.KV_FP8, 4, 16, 1, True, gen.Q_BF16, 1.0),
    (gen.KV_BF16, 2, 32, 4, False, gen.Q_BF16, 1.0), (gen.KV_FP8, 3, 8, 2, True, gen.Q_BF16, 1.0),
    (gen.KV_E5M2, 1, 64, 4, True, gen.Q_BF16, 1.0), (gen.KV_FP8, 1, 64, 4, False, gen.Q_FP8, 0.5),
    (gen.KV_FP8, 4, 16, 1, True, gen.Q_FP8, 1.0), (gen.KV_E5M2, 2, 32, 4, False, gen.Q_FP8, 2.0),
    (gen.KV_MXFP4, 2, 16, 1, True, gen.Q_BF16, 1.0), (gen.KV_MXFP4, 1, 64, 4, False, gen.Q_FP8, 0.5)])
def test_scorer_matches_oracle(kvd, dql, hq, hkv, transposed, qd, qs):
    _banner(f"scorer kv={kvd} q={qd} q_scale={qs} dql={dql} heads=({hq},{hkv}) "
            f"transposed={transposed}")
    case = gen.make_random_case(121, 3, dql, hq, hkv, 16, 100, 3000, kv_dtype=kvd, pad_rows=2,
                                q_dtype=qd, q_scale=qs)
    case.k_scale = 0.75
    d = DevCase(case)
    mb = case.max_blocks + 2
    score, _ = _run_scorer(d, mb, 16, transposed)
    ref = oracle_scores(case, mb)
    _scores_close(score[:, :, :case.real_rows], ref, case)
    assert np.all(np.isneginf(score[:, :, case.real_rows:]))


@pytest.mark.parametrize("name,transposed", [("c2_tp4_fp8", True), ("c3_tp1_fp8", False),
                                              ("bf16_long", True)])
def test_scorer_full_size_sampled_rows(name, transposed):
    """Scores of long sequences, where every workgroup of the persistent scorer
    walks many blocks across request and head boundaries: all cells are
    checked for -inf placement and sampled token rows against the oracle."""
    _banner(f"scorer full size {name} transposed={transposed}")
    if name == "bf16_long":
        case = gen.make_random_case(141, 6, 2, 16, 2, 16, 60000, 131072, kv_dtype=gen.KV_BF16,
                                    pad_rows=3)
    else:
        case = gen.make_config(name)
    d = DevCase(case)
    mb = case.max_blocks
    score, _ = _run_scorer(d, mb, 16, transposed)
    pos = case.positions()
    visible = np.arange(mb)[None, :] * 128 <= pos[:, None]                 # [rows, mb]
    for h in range(case.num_kv_heads):
        assert np.array_equal(np.isneginf(score[h, :, :case.real_rows]), ~visible.T)
    assert np.all(np.isneginf(score[:, :, case.real_rows:]))
    rng = np.random.default_rng(7)
    rows = sorted(set(rng.choice(case.real_rows, 4, replace=False).tolist()
                      + [case.real_rows - 1]))
    ref = oracle_scores(case, mb, rows=rows)
    _scores_close(score[:, :, rows], ref)


@pytest.mark.parametrize("tie_frac,transposed,k", [(0.0, False, 16), (0.4, False, 16),
                                                   (0.4, True, 5), (0.0, True, 64)])
def test_selector_bit_exact_on_given_scores(tie_frac, transposed, k):
    _banner(f"selector ties={tie_frac} transposed={transposed} k={k}")
    seq = np.array([129, 700, 5000, 20000], dtype=np.int32)
    nb = 160
    sc = gen.make_scores(131, 3, nb, 8, seq, 2, tie_frac=tie_frac)
    if transposed:
        dev = torch.from_numpy(np.ascontiguousarray(sc.transpose(0, 2, 1))).cuda().transpose(1, 2)
    else:
        dev = torch.from_numpy(sc).cuda()
    out = torch.full((8, 3, k), -7, dtype=torch.int32, device="cuda")
    msa.msa_topk_select(dev, out)
    torch.cuda.synchronize()
    ref = om.select_topk(sc.astype(np.float64), k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("nb,k", [(2048, 16), (8000, 64), (16384, 7)])
def test_selector_long_rows(nb, k):
    """Rows of up to 16384 blocks (every per-thread register width of the
    selector), with planted ties."""
    _banner(f"selector long rows nb={nb} k={k}")
    seq = np.array([nb * 128, nb * 64, 3 * 128 + 5], dtype=np.int32)
    sc = gen.make_scores(151, 2, nb, 3, seq, 1, tie_frac=0.3)
    dev = torch.from_numpy(np.ascontiguousarray(sc.transpose(0, 2, 1))).cuda().transpose(1, 2)
    out = torch.full((3, 2, k), -7, dtype=torch.int32, device="cuda")
    msa.msa_topk_select(dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), om.select_topk(sc.astype(np.float64), k))


def test_selector_special_values():
    """+-0 rank as equal (ties to the lower block), +inf is selectable, -inf and
    NaN never are, subnormals and the extreme finite values keep their order."""
    _banner("selector special values")
    vals = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40,
                     -1e-40, 2.0], dtype=np.float32)
    rng = np.random.default_rng(161)
    sc = rng.choice(vals, size=(2, 300, 5)).astype(np.float32)
    sc[1, :, 4] = np.nan                       # a row with nothing selectable
    sc[0, :, 3] = -0.0
    sc[0, 7, 3] = 0.0                          # all equal once -0 == +0
    dev = torch.from_numpy(sc).cuda()
    for k in (1, 16, 64):
        out = torch.full((5, 2, k), -7, dtype=torch.int32, device="cuda")
        msa.msa_topk_select(dev, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), om.select_topk(sc.astype(np.float64), k)), k


@pytest.mark.parametrize("k", [1, 16, 64])
def test_selector_prefilter_and_radix_fallback(k):
    """Rows whose candidate set (blocks at or above the k-th largest
    per-thread maximum) stays small take the compare-and-rank path; rows
    where ties leave more than 512 candidates (all 2048 equal, 600 tied at the
    top, 600 tied at the k-th place) take the radix select.  Both must equal
    the oracle's ranking, ties going to the lower block."""
    _banner(f"selector prefilter / radix fallback k={k}")
    rng = np.random.default_rng(171)
    nb, rows = 2048, 8
    sc = rng.standard_normal((1, nb, rows)).astype(np.float32)
    sc[0, :, 1] = 0.5                                        # all equal: fallback
    top = rng.choice(nb, 600, replace=False)
    sc[0, top, 2] = 9.0                                      # 600 tied at the top
    sc[0, :, 3] = rng.standard_normal(nb).astype(np.float32) - 10.0
    sc[0, top[:k - 1], 3] = 5.0                              # k-1 clear winners ...
    sc[0, top[k - 1:], 3] = 4.0                              # ... then 600-k+1 tied
    tie = rng.choice(nb, 400, replace=False)
    sc[0, tie, 4] = 7.0                                      # 400 tied: fast path
    sc[0, :, 5] = np.round(sc[0, :, 5] * 2) / 2              # coarse ties
    sc[0, rng.random(nb) < 0.9, 6] = -np.inf                 # ~200 selectable
    sc[0, :, 7] = -np.inf
    sc[0, :5, 7] = 1.0                                       # fewer than k selectable
    dev = torch.from_numpy(np.ascontiguousarray(sc.transpose(0, 2, 1))).cuda().transpose(1, 2)
    out = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    msa.msa_topk_select(dev, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), om.select_topk(sc.astype(np.float64), k))


def _gap_ok_rows(ref_scores, k, eps):
    """(t, h) pairs whose oracle k-th and (k+1)-th scores differ by > eps."""
    hkv, nb, nt = ref_scores.shape
    ok = np.zeros((nt, hkv), dtype=bool)
    for h in range(hkv):
        for t in range(nt):
            s = np.sort(ref_scores[h, :, t][np.isfinite(ref_scores[h, :, t])])[::-1]
            if len(s) <= k:
                ok[t, h] = True
            else:
                ok[t, h] = (s[k - 1] - s[k]) > eps and np.all(np.diff(s[:k + 1]) != 0)
    return ok


def _same_picks(sel, ref_sel, ok, score, what):
    """On the (row, kv head) pairs `ok`, the GPU's picks are the oracle's
    blocks, -1 padding included, ranked by the GPU's own scores (non-increasing;
    the selector's order itself is checked bit for bit on given scores)."""
    assert np.array_equal(np.sort(sel[ok], axis=-1), np.sort(ref_sel[ok], axis=-1)), \
        f"{what}: selected blocks"
    for t, h in zip(*np.nonzero(ok)):
        picks = sel[t, h][sel[t, h] >= 0]
        assert np.all(np.diff(score[h, picks, t]) <= 0), (what, t, h, picks)


def _attend_over_oracle_selection(case, mb, score, sel, got, k, what):
    """The oracle's own scores and top-k for every real row, then its attend
    over that top-k.  The GPU's scores must lie within the scorer's bound and
    its selection must hold the oracle's blocks wherever the top-k has a clear
    gap (in the order of its own scores: two picks closer than the scorer's
    error may rank either way);
    the GPU output `got` is compared with the oracle's on the q heads of those
    (row, kv head) pairs.  Every oracle input comes from the case or the
    oracle itself, never from the GPU."""
    real = case.real_rows
    ref_scores = oracle_scores(case, mb)
    tol = _scores_close(score[:, :, :real], ref_scores, case)
    ref_sel = om.select_topk(ref_scores, k)
    ok = _gap_ok_rows(ref_scores, k, 4 * tol)
    _same_picks(sel[:real], ref_sel, ok, score, what)
    # Which pairs have a clear gap depends only on the oracle's scores and the
    # bound.  The fp8-q bound is a worst case (about 200x the error measured),
    # under which a quarter to a third of these pairs keep one; the floor only
    # keeps the comparison from being vacuous.
    assert ok.mean() > (0.2 if case.q_dtype == gen.Q_FP8 else 0.8), ok.mean()
    ref = oracle_attend(case, rows=list(range(real)), topk=ref_sel)
    mask = np.repeat(ok, case.num_q_heads // case.num_kv_heads, axis=1)
    assert_parity(got[:real][mask], ref[mask], what=what)
    return ok


@pytest.mark.parametrize("kvd,qd,qs", [(gen.KV_FP8, gen.Q_BF16, 1.0),
                                       (gen.KV_FP8, gen.Q_FP8, 0.5),
                                       (gen.KV_E5M2, gen.Q_BF16, 1.0),
                                       (gen.KV_MXFP4, gen.Q_BF16, 1.0),
                                       (gen.KV_MXFP4, gen.Q_FP8, 0.5)])
def test_full_step_score_select_attend(kvd, qd, qs):
    _banner(f"full step: score -> top-16 -> attend, kv={kvd} q={qd}")
    case = gen.make_random_case(141, 6, 1, 64, 4, 16, 3000, 30000, kv_dtype=kvd, q_dtype=qd,
                                q_scale=qs)
    d = DevCase(case)
    mb = case.max_blocks
    score, sel = _run_scorer(d, mb, 16)
    ref_scores = oracle_scores(case, mb)
    tol = _scores_close(score[:, :, :case.real_rows], ref_scores, case)
    ref_sel = om.select_topk(ref_scores, 16)
    ok = _gap_ok_rows(ref_scores, 16, 4 * tol)
    # Rows with a clear top-16 / 17th gap must match exactly; the rest are
    # checked for validity below.  Which units have a clear gap depends only
    # on the oracle's scores and the error bound, not on the GPU: with a bf16
    # q (bound 2e-5 of the largest score) 23 or 24 of the 24 (row, head)
    # units do on these inputs; the fp8-q bound is a worst case (~200x the
    # error measured here), under which 14 (e4m3) and 10 (MXFP4) do.
    assert ok.mean() > (0.3 if qd == gen.Q_FP8 else 0.8)
    assert np.array_equal(sel[ok], ref_sel[ok])
    # Rows without a clear gap get a valid top-16 by the oracle's scores:
    # distinct visible blocks, -1 only as trailing padding and only when
    # fewer than 16 blocks are visible, in non-increasing score order up to
    # twice the bound (the GPU ranks by its own scores), and each pick within
    # the bound of the oracle's 16th best.
    for t, h in zip(*np.nonzero(~ok)):
        row = ref_scores[h, :, t]
        n_vis = int(np.isfinite(row).sum())
        picks = sel[t, h]
        n_sel = int((picks >= 0).sum())
        assert n_sel == min(16, n_vis), (t, h, picks)
        assert np.all(picks[:n_sel] >= 0) and np.all(picks[n_sel:] == -1), (t, h, picks)
        got_b = picks[:n_sel]
        assert len(np.unique(got_b)) == n_sel, (t, h, picks)
        assert np.all(np.isfinite(row[got_b])), (t, h, picks)
        assert np.all(np.diff(row[got_b]) <= 2 * tol), (t, h, picks)
        kth = np.sort(row[np.isfinite(row)])[::-1][n_sel - 1]
        assert np.all(row[got_b] >= kth - 4 * tol), (t, h, picks)
    # Attend over the GPU's own selection, compared where it equals the oracle's.
    case.topk = ref_sel
    out = d.new_out()
    d.run(d.plan(), topk=torch.from_numpy(sel).cuda(), out=out)
    torch.cuda.synchronize()
    rows = [t for t in range(case.real_rows) if ok[t].all()]
    assert_parity(to_f64(out)[rows], oracle_attend(case, rows=rows), what="full step")


def test_full_step_at_the_largest_scorer_batch():
    """The scorer's largest batch, 4096 requests (its LDS prefix sum over the
    requests' block counts is sized for it), of 1..400 tokens each; then the
    attend of the scorer's top-4 over 4096 units, and the selecting attend,
    which must equal it bit for bit.  Scores, selection and output are checked
    against the oracle on every row (selection and output where the top-4
    has a clear gap)."""
    _banner("full step at batch 4096 (scorer limit), seq 1..400, top-4")
    case = gen.make_random_case(161, 4096, 1, 16, 1, 4, 1, 400)
    d = DevCase(case)
    mb = case.max_blocks
    score, sel = _run_scorer(d, mb, 4)
    out = d.new_out()
    plan = d.plan()
    d.run(plan, topk=torch.from_numpy(sel).cuda(), out=out)
    got = d.new_out()
    sel2 = torch.full((case.num_token_rows, 1, 4), -7, dtype=torch.int32, device="cuda")
    msa.msa_sparse_decode_select_run(plan, d.q, d.kv, d.block_table, d.seq_lens,
                                     torch.from_numpy(score.astype(np.float32)).cuda(), got,
                                     topk_out=sel2, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(sel2.cpu().numpy(), sel)
    assert torch.equal(got.view(torch.int16), out.view(torch.int16))
    _attend_over_oracle_selection(case, mb, score, sel, to_f64(out), 4, "batch 4096")


def test_scorer_at_the_largest_query_length():
    """decode_query_len 32, the scorer's largest: 32 token rows per request,
    each with its own causal limit, scored against the oracle on every row;
    the top-16 bit-exact where it has a clear gap."""
    _banner("scorer at dql=32 (scorer limit), heads (64,4)")
    case = gen.make_random_case(162, 3, 32, 64, 4, 16, 2000, 9000, pad_rows=2)
    d = DevCase(case)
    mb = case.max_blocks + 1
    score, sel = _run_scorer(d, mb, 16)
    ref = oracle_scores(case, mb)
    tol = _scores_close(score[:, :, :case.real_rows], ref, case)
    assert np.all(np.isneginf(score[:, :, case.real_rows:]))
    ok = _gap_ok_rows(ref, 16, 4 * tol)
    assert ok.mean() > 0.8
    _same_picks(sel[:case.real_rows], om.select_topk(ref, 16), ok, score, "dql 32")
    assert np.all(sel[case.real_rows:] == -1)


@pytest.mark.parametrize("tile_rows,splits", [(1, 1), (1, 2), (1, 4), (1, 6), (1, 16),
                                               (2, 3), (2, 8), (4, 5)])
def test_attend_then_merge_equals_run(tile_rows, splits):
    """The two halves of a run equal the run, bitwise, for the fused in-attend
    merge (single-row, 2..4 splits), the merge kernel's unrolled counts and
    its generic loop (6 and 5 splits), and row-tile plans (which always merge
    in a second launch); the merged rows also match the oracle."""
    _banner(f"attend + merge == run, tile_rows={tile_rows} splits={splits}")
    case = gen.make_random_case(115, 4, 4, 16, 1, 16, 2000, 20000, pad_rows=2)
    d = DevCase(case)
    ref = oracle_attend(case)
    plan = d.plan(splits, tile_rows=tile_rows)
    assert (plan.num_splits, plan.tile_rows) == (splits, tile_rows)
    a = d.new_out()
    b = d.new_out()
    d.run(plan, out=a)
    msa.msa_sparse_decode_attend(plan, d.q, d.kv, d.block_table, d.seq_lens, d.topk, b,
                                 sm_scale=case.sm_scale, k_scale=case.k_scale,
                                 v_scale=case.v_scale)
    msa.msa_sparse_decode_merge(plan, b, v_scale=case.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_parity(to_f64(b), ref, what=f"attend + merge, {splits} splits")


def test_fused_merge_counters_return_to_zero():
    """Single-row plans with 2..4 splits merge inside the attend through
    per-unit arrival counters that every run leaves at zero: repeated eager
    runs with changing inputs, then a captured graph replayed with eager runs
    in between, each checked against the oracle (a counter left non-zero
    would skip or double a combine)."""
    _banner("fused split merge: repeated runs and graph replays")
    case = gen.make_random_case(117, 6, 2, 16, 2, 8, 500, 9000, pad_rows=1)
    other = gen.make_random_case(117, 6, 2, 16, 2, 8, 500, 9000, pad_rows=1)
    other.q = gen.make_q(np.random.default_rng(5), other.num_token_rows, other.num_q_heads)
    refs = [oracle_attend(case), oracle_attend(other)]
    q_sets = [torch.from_numpy(c.q.view(np.int16)).view(torch.bfloat16).cuda()
              for c in (case, other)]
    d = DevCase(case)
    for splits in (2, 3, 4):
        plan = d.plan(splits)
        assert plan.merges_in_attend and plan.num_splits == splits
        for rep in range(4):
            d.q.copy_(q_sets[rep % 2])
            out = d.new_out()
            d.run(plan, out=out)
            torch.cuda.synchronize()
            assert_parity(to_f64(out), refs[rep % 2], what=f"splits={splits} run {rep}")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            d.run(plan)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            d.run(plan)
        for rep in range(3):
            d.q.copy_(q_sets[rep % 2])
            d.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert_parity(to_f64(d.out), refs[rep % 2], what=f"splits={splits} replay {rep}")
            eager = d.new_out()
            d.q.copy_(q_sets[(rep + 1) % 2])
            d.run(plan, out=eager)
            torch.cuda.synchronize()
            assert_parity(to_f64(eager), refs[(rep + 1) % 2], what=f"eager between {rep}")


def test_indexer_step_graph_replays():
    """The indexer step (block-max scores, top-k) and the attend over its
    selection captured in one graph, replayed with q changed in place and an
    eager step between replays; every replay's scores, selections and output
    are checked (scores against the oracle, selections on rows with a clear
    score gap, the output against the oracle fed the GPU's selection)."""
    _banner("indexer step in a graph: replays")
    case = gen.make_random_case(118, 4, 1, 32, 2, 16, 3000, 20000)
    qs = [case.q, gen.make_q(np.random.default_rng(8), case.num_token_rows, case.num_q_heads)]
    q_dev = [torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda() for q in qs]
    d = DevCase(case)
    mb = case.max_blocks
    rows = case.num_token_rows
    score = torch.full((case.num_kv_heads, mb, rows), float("nan"), device="cuda")
    sel = torch.full((rows, case.num_kv_heads, 16), -7, dtype=torch.int32, device="cuda")
    plan = d.plan()

    def step(out):
        d.score(score, sel, mb, num_token_rows=rows)
        d.run(plan, topk=sel, out=out)

    def check(out, qi, what):
        c = gen.make_random_case(118, 4, 1, 32, 2, 16, 3000, 20000)
        c.q = qs[qi]
        _attend_over_oracle_selection(c, mb, score.cpu().numpy().astype(np.float64),
                                      sel.cpu().numpy(), to_f64(out), 16, what)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(d.out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(d.out)
    for rep in range(3):
        qi = rep % 2
        d.q.copy_(q_dev[qi])
        d.out.fill_(float("nan"))
        score.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(d.out, qi, f"replay {rep}")
        eager = d.new_out()
        d.q.copy_(q_dev[1 - qi])
        step(eager)
        torch.cuda.synchronize()
        check(eager, 1 - qi, f"eager between {rep}")


def test_c5_full_step_full_size_sampled_rows():
    """The full decode step with the indexer at full size (B=64, 64/4 heads,
    seq up to 262144): GPU scores, top-16 and attend checked on sampled token
    rows that the oracle evaluates one by one."""
    _banner("c5 full step, full size")
    case = gen.make_config("c5_full_step")
    d = DevCase(case)
    mb = case.max_blocks
    rows_all = case.num_token_rows
    # the timed layout: physical [Hkv, rows, blocks] seen as logical [Hkv, blocks, rows]
    score = torch.full((case.num_kv_heads, rows_all, mb), float("nan"),
                       device="cuda").transpose(1, 2)
    sel = torch.full((rows_all, case.num_kv_heads, 16), -7, dtype=torch.int32, device="cuda")
    msa.msa_block_score_topk(d.q, d.kv, d.block_table, d.seq_lens, decode_query_len=case.dql,
                             num_kv_heads=case.num_kv_heads, max_blocks=mb, score=score,
                             topk_out=sel, k_scale=case.k_scale)
    out = d.new_out()
    plan = msa.msa_sparse_decode_plan(
        case.batch, case.dql, num_q_heads=case.num_q_heads, num_kv_heads=case.num_kv_heads,
        page_table_stride=d.block_table.stride(0), topk_blocks=16, kv_dtype=msa.KV_FP8_E4M3,
        device=d.dev)
    msa.msa_sparse_decode_run(plan, d.q, d.kv, d.block_table, d.seq_lens, sel, out,
                              sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    # the longest and shortest requests plus random ones
    order = np.argsort(case.seq_lens)
    rows = sorted(set([int(order[0]), int(order[-1])] + rng.choice(64, 4, replace=False).tolist()))
    ref_scores = om.block_max_scores(case.q, case.kv, case.kv_dtype, case.k_scale,
                                     case.block_table, case.seq_lens, case.dql,
                                     case.num_kv_heads, mb, rows=rows)
    got_scores = score.cpu().numpy().astype(np.float64)[:, :, rows]
    tol = _scores_close(got_scores, ref_scores)
    ref_sel = om.select_topk(ref_scores, 16)                      # [len(rows), Hkv, 16]
    got_sel = sel.cpu().numpy()[rows]
    ok = _gap_ok_rows(ref_scores, 16, 4 * tol)
    assert ok.mean() > 0.8
    assert np.array_equal(got_sel[ok], ref_sel[ok])
    full_sel = np.full_like(sel.cpu().numpy(), -1)      # the oracle reads only `rows`
    for i, t in enumerate(rows):
        full_sel[t] = ref_sel[i]
    ok_rows = [t for i, t in enumerate(rows) if ok[i].all()]
    assert ok_rows
    ref_out = oracle_attend(case, rows=ok_rows, topk=full_sel)
    assert_parity(to_f64(out)[ok_rows], ref_out, what=f"c5 attend on {len(ok_rows)} rows")


@pytest.mark.parametrize("kvd,qd,qs,splits,mb_extra", [
    (gen.KV_FP8, gen.Q_BF16, 1.0, 1, 0),
    (gen.KV_FP8, gen.Q_BF16, 1.0, 2, 0),        # the in-attend split merge
    (gen.KV_FP8, gen.Q_FP8, 0.5, 8, 0),         # the merge kernel
    (gen.KV_E5M2, gen.Q_BF16, 1.0, 3, 0),
    (gen.KV_MXFP4, gen.Q_FP8, 0.5, 1, 0),
    (gen.KV_FP8, gen.Q_BF16, 1.0, 1, 2100),     # more than 2048 score columns
])
def test_select_run_equals_select_then_run(kvd, qd, qs, splits, mb_extra):
    """msa_sparse_decode_select_run selects each row's top-k from the scores
    inside the attend: its output and selection equal, bit for bit, the
    selector's top-k fed to msa_sparse_decode_run (padding rows: zeros and
    all -1), and the rows match the oracle over that selection."""
    _banner(f"select_run kv={kvd} q={qd} splits={splits} extra columns={mb_extra}")
    case = gen.make_random_case(143, 5, 2, 64, 4, 16, 1500, 40000, kv_dtype=kvd, q_dtype=qd,
                                q_scale=qs, pad_rows=3)
    d = DevCase(case)
    mb = case.max_blocks + mb_extra
    rows = case.num_token_rows
    score = torch.full((case.num_kv_heads, mb, rows), float("nan"), device="cuda")
    sel = torch.full((rows, case.num_kv_heads, 16), -7, dtype=torch.int32, device="cuda")
    d.score(score, sel, mb, num_token_rows=rows)
    plan = d.plan(splits, tile_rows=1)
    assert plan.num_splits == splits
    ref = d.new_out()
    d.run(plan, topk=sel, out=ref)
    got = d.new_out()
    sel2 = torch.full_like(sel, -7)
    msa.msa_sparse_decode_select_run(plan, d.q, d.kv, d.block_table, d.seq_lens, score, got,
                                     topk_out=sel2, sm_scale=case.sm_scale,
                                     k_scale=case.k_scale, v_scale=case.v_scale,
                                     q_scale=case.q_scale)
    torch.cuda.synchronize()
    assert torch.equal(sel2, sel)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert np.all(to_f64(got)[case.real_rows:] == 0.0)
    _attend_over_oracle_selection(case, mb, score.cpu().numpy().astype(np.float64),
                                  sel.cpu().numpy(), to_f64(got), 16, "select_run rows")


def test_select_run_rows_longer_than_the_staged_table():
    """Rows of more than 2048 blocks: the selecting attend stages only the
    first 2048 block-table entries of a request, and reads the entries of
    later selected blocks from the table itself.  Equal, bit for bit, to the
    selector's top-k fed to msa_sparse_decode_run, and to the oracle."""
    _banner("select_run rows past the staged table (seq 270k..300k)")
    case = gen.make_random_case(145, 2, 2, 16, 1, 16, 270000, 300000, pad_rows=1)
    d = DevCase(case)
    mb = case.max_blocks
    assert mb > 2048
    rows = case.num_token_rows
    score = torch.full((1, mb, rows), float("nan"), device="cuda")
    sel = torch.full((rows, 1, 16), -7, dtype=torch.int32, device="cuda")
    d.score(score, sel, mb, num_token_rows=rows)
    plan = d.plan(1, tile_rows=1)
    ref = d.new_out()
    d.run(plan, topk=sel, out=ref)
    got = d.new_out()
    sel2 = torch.full_like(sel, -7)
    msa.msa_sparse_decode_select_run(plan, d.q, d.kv, d.block_table, d.seq_lens, score, got,
                                     topk_out=sel2, sm_scale=case.sm_scale)
    torch.cuda.synchronize()
    picked = sel.cpu().numpy()
    assert (picked[: case.real_rows] >= 2048).any(), "no selected block past the staged entries"
    assert torch.equal(sel2, sel)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    ok = _attend_over_oracle_selection(case, mb, score.cpu().numpy().astype(np.float64),
                                       picked, to_f64(got), 16, "select_run long rows")
    assert (picked[: case.real_rows][ok] >= 2048).any(), "no compared pick past 2048"
    assert np.all(to_f64(got)[case.real_rows:] == 0.0)


def test_select_run_in_a_graph_with_new_scores():
    """Captured once, replayed with the score buffer rewritten in place: every
    replay selects from the scores it finds (the selection equals the
    selector's on the same scores)."""
    _banner("select_run graph replay")
    case = gen.make_random_case(144, 4, 1, 16, 1, 16, 3000, 20000)
    d = DevCase(case)
    mb = case.max_blocks
    rows = case.num_token_rows
    score = torch.full((1, mb, rows), float("nan"), device="cuda")
    sel = torch.full((rows, 1, 16), -7, dtype=torch.int32, device="cuda")
    d.score(score, sel, mb, num_token_rows=rows)
    torch.cuda.synchronize()
    plan = d.plan(2, tile_rows=1)
    out = d.new_out()
    got_sel = torch.full_like(sel, -7)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        msa.msa_sparse_decode_select_run(plan, d.q, d.kv, d.block_table, d.seq_lens, score,
                                         out, topk_out=got_sel, sm_scale=case.sm_scale,
                                         stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        msa.msa_sparse_decode_select_run(plan, d.q, d.kv, d.block_table, d.seq_lens, score,
                                         out, topk_out=got_sel, sm_scale=case.sm_scale)
    rng = np.random.default_rng(7)
    finite = torch.isfinite(score)
    for rep in range(3):
        noise = torch.from_numpy(rng.standard_normal(tuple(score.shape)).astype(np.float32))
        score.copy_(torch.where(finite, noise.cuda(), score))
        ref_sel = torch.full_like(sel, -7)
        msa.msa_topk_select(score, ref_sel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got_sel, ref_sel), rep
        ref = d.new_out()
        d.run(d.plan(2, tile_rows=1), topk=ref_sel, out=ref)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
