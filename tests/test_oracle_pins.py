"""Pins for the float64 oracle (CPU only).

Each check ties the oracle to something other than itself: torch's own fp8 /
bf16 casts, dense causal attention computed by
``torch.nn.functional.scaled_dot_product_attention`` on the un-paged sequence,
closed forms, invariances, brute-force loops and hand-worked values from the
pages (``tests/golden/page_facts.json``).  The last group plants plausible
mistakes in the oracle's helpers and checks that a pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.msa_oracle as om
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# independent reference helpers (torch casts, SDPA)
# ---------------------------------------------------------------------------

def torch_values(kv: np.ndarray, kv_dtype: str) -> torch.Tensor:
    """Decode the stored entries with torch's own dtype casts (float64)."""
    if kv_dtype == gen.KV_FP8:
        return torch.from_numpy(np.ascontiguousarray(kv)).view(torch.float8_e4m3fn).to(
            torch.float64)
    if kv_dtype == gen.KV_E5M2:
        return torch.from_numpy(np.ascontiguousarray(kv)).view(torch.float8_e5m2).to(
            torch.float64)
    return torch.from_numpy(np.ascontiguousarray(kv).view(np.int16)).view(
        torch.bfloat16).to(torch.float64)


def torch_q(q_bits: np.ndarray, q_dtype: str = gen.Q_BF16, q_scale: float = 1.0
            ) -> torch.Tensor:
    """q values through torch's casts: bf16 bits, or e4m3fn codes, times q_scale
    (the test page feeds its reference ``query_fp8.to(bfloat16) * q_scale``)."""
    if q_dtype == gen.Q_FP8:
        v = torch.from_numpy(np.ascontiguousarray(q_bits)).view(torch.float8_e4m3fn)
    else:
        v = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(
            torch.bfloat16)
    return v.to(torch.float64) * q_scale


def dense_reference(case: gen.DecodeCase, values=None) -> np.ndarray:
    """Textbook causal GQA attention over each request's whole (un-paged)
    sequence, via SDPA in float64.  Equals the sparse attend when the index
    lists cover every visible block.  ``values`` (float [blocks, Hkv, 128,
    256], K|V before the per-tensor scales) replaces torch's decode of the
    stored entries, for a cache built from known values."""
    hq, hkv = case.num_q_heads, case.num_kv_heads
    g = hq // hkv
    vals = (torch_values(case.kv, case.kv_dtype) if values is None
            else torch.from_numpy(np.asarray(values, dtype=np.float64)))
    q = torch_q(case.q, case.q_dtype, case.q_scale)
    out = torch.zeros(case.num_token_rows, hq, 128, dtype=torch.float64)
    for r in range(case.batch):
        s = int(case.seq_lens[r])
        n = gen.pages_for(s)
        pages = torch.from_numpy(case.block_table[r, :n].astype(np.int64))
        seqkv = vals[pages].permute(1, 0, 2, 3).reshape(hkv, n * 128, 256)[:, :s]
        k = (seqkv[..., :128] * case.k_scale).repeat_interleave(g, dim=0)
        v = (seqkv[..., 128:] * case.v_scale).repeat_interleave(g, dim=0)
        t0 = r * case.dql
        qh = q[t0:t0 + case.dql].permute(1, 0, 2)
        pos = s - case.dql + torch.arange(case.dql)
        mask = torch.arange(s)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qh, k, v, attn_mask=mask, scale=case.sm_scale)
        out[t0:t0 + case.dql] = o.permute(1, 0, 2)
    return out.numpy()


def run_oracle(case: gen.DecodeCase, topk=None, **over) -> np.ndarray:
    kw = dict(q_bits=case.q, kv=case.kv, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
              v_scale=case.v_scale, block_table=case.block_table, seq_lens=case.seq_lens,
              topk=case.topk if topk is None else topk, decode_query_len=case.dql,
              num_kv_heads=case.num_kv_heads, sm_scale=case.sm_scale,
              q_dtype=case.q_dtype, q_scale=case.q_scale)
    kw.update(over)
    return om.sparse_decode(**kw)


def dense_pin_error(case: gen.DecodeCase) -> float:
    got = run_oracle(case)
    ref = dense_reference(case)
    return float(np.max(np.abs(got - ref)))


def small_dense_case(hq=16, hkv=1, dql=4, kv_dtype=gen.KV_FP8, pattern=(257, 513),
                     pairs=1, seed=0, k_scale=1.0, v_scale=1.0, q_dtype=gen.Q_BF16,
                     q_scale=1.0):
    case = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=pattern, seed=seed,
                            kv_dtype=kv_dtype, topk_k=8, q_dtype=q_dtype, q_scale=q_scale)
    case.k_scale, case.v_scale = k_scale, v_scale
    return case


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_e4m3fn_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = om.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.all(both_nan | (mine == ref))
    # sign of zero too
    assert np.array_equal(np.signbit(mine[~both_nan]), np.signbit(ref[~both_nan]))


def test_e5m2_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = om.decode_e5m2(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])           # includes +-inf
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))
    fin = np.isfinite(mine)
    assert np.max(mine[fin]) == 57344.0 and np.sum(np.isinf(mine)) == 2


def test_e4m3fn_golden_codes():
    g = golden()["e4m3fn"]
    for code, val in g["codes"].items():
        assert om.decode_e4m3fn(np.array([int(code, 16)]))[0] == val, code
    nan = {int(c, 16) for c in g["nan_codes"]}
    vals = om.decode_e4m3fn(np.arange(256))
    assert set(np.nonzero(np.isnan(vals))[0].tolist()) == nan
    assert np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = om.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_dequant_applies_scale():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    assert np.array_equal(om.dequant(codes, "fp8_e4m3", 0.5), om.decode_e4m3fn(codes) * 0.5)
    codes = np.arange(0, 0x7C, dtype=np.uint8)
    assert np.array_equal(om.dequant(codes, "fp8_e5m2", 0.25), om.decode_e5m2(codes) * 0.25)


def test_fp8_query_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = om.decode_query(codes, "fp8_e4m3", 0.5)
    ref = torch_q(codes, gen.Q_FP8, 0.5).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


# ---------------------------------------------------------------------------
# page-fixed facts
# ---------------------------------------------------------------------------

def test_visible_pages_match_test_page_formula():
    for c in golden()["visible_pages"]["cases"]:
        s, ql = c["seq_len"], c["query_len"]
        got = []
        for loc in range(ql):
            pos = om.token_position(s, ql, loc)
            got.append(sum(1 for b in range(64) if om.visible_rows(pos, b) > 0))
        assert got == c["pages"], c


def test_generator_stride_and_scale_facts():
    g = golden()
    case = gen.make_p3_case(64, 4, 1, 1, seed=0, poison=False)
    strides = [s // case.kv.itemsize for s in case.kv.strides]
    assert strides == g["kv_cache_strides_hnd"]["num_kv_heads_4"]
    assert case.sm_scale == g["sm_scale"]["value"]
    case1 = gen.make_p3_case(16, 1, 1, 1, seed=0, poison=False)
    assert [s // case1.kv.itemsize for s in case1.kv.strides] == \
        g["kv_cache_strides_hnd"]["num_kv_heads_1"]


# ---------------------------------------------------------------------------
# attend == dense causal attention when every visible block is selected
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dql", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("heads", [(16, 1), (8, 2)])
@pytest.mark.parametrize("kv_dtype", [gen.KV_FP8, gen.KV_BF16])
def test_dense_equivalence(dql, heads, kv_dtype):
    case = small_dense_case(heads[0], heads[1], dql, kv_dtype)
    assert dense_pin_error(case) < 1e-12


@pytest.mark.parametrize("dql", [1, 4])
@pytest.mark.parametrize("fmt", [(gen.KV_E5M2, gen.Q_BF16, 1.0), (gen.KV_FP8, gen.Q_FP8, 1.0),
                                 (gen.KV_FP8, gen.Q_FP8, 0.5), (gen.KV_E5M2, gen.Q_FP8, 0.25)])
def test_dense_equivalence_other_formats(dql, fmt):
    """e5m2 KV and fp8 q with a q scale, against SDPA on torch-decoded values."""
    kv_dtype, q_dtype, q_scale = fmt
    case = small_dense_case(8, 2, dql, kv_dtype, q_dtype=q_dtype, q_scale=q_scale)
    assert dense_pin_error(case) < 1e-12


def test_q_scale_is_a_softmax_temperature():
    """softmax(c * (s q) . k) == softmax((c s) q . k): a q scale acts exactly
    like the same factor on sm_scale (the definition, reading 9)."""
    case = small_dense_case(8, 2, 3, q_dtype=gen.Q_FP8, q_scale=0.75)
    a = run_oracle(case)
    b = run_oracle(case, q_scale=1.0, sm_scale=case.sm_scale * 0.75)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("pattern", [(129, 385), (1, 128), (127, 130)])
def test_dense_equivalence_boundaries(pattern):
    case = small_dense_case(8, 2, 2 if min(pattern) > 1 else 1, pattern=pattern)
    assert dense_pin_error(case) < 1e-12


def test_dense_equivalence_with_scales():
    case = small_dense_case(8, 2, 3, k_scale=0.5, v_scale=2.0)
    assert dense_pin_error(case) < 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _const_v_case(code):
    case = small_dense_case(8, 2, 4)
    kv = case.kv.copy()
    kv[..., 128:] = code
    case.kv = kv
    return case


def test_constant_v_gives_that_value():
    code = 0x3C  # 1.5
    case = _const_v_case(code)
    case.v_scale = 2.0
    # the tails past seq_len were overwritten too, but they must stay invisible:
    out = run_oracle(case)
    assert np.allclose(out, 3.0, rtol=0, atol=1e-12)


def test_single_visible_key():
    # dql = 1, seq = b*128 + 1: token position b*128 sees exactly one key of
    # block b; selecting only block b gives that key's V.
    case = gen.make_p3_case(16, 1, 1, 1, seq_pattern=(3 * 128 + 1,), seed=3)
    topk = np.full_like(case.topk, -1)
    topk[0, 0, 0] = 3
    out = run_oracle(case, topk=topk)
    p = case.block_table[0, 3]
    v = torch_values(case.kv[p, 0, 0, 128:], case.kv_dtype).numpy() * case.v_scale
    assert np.allclose(out[0], v[None, :], rtol=0, atol=1e-15)


def test_seq_len_one():
    case = gen.make_p3_case(16, 1, 1, 1, seq_pattern=(1,), seed=4)
    out = run_oracle(case)
    p = case.block_table[0, 0]
    v = torch_values(case.kv[p, 0, 0, 128:], case.kv_dtype).numpy()
    assert np.allclose(out[0], v[None, :], rtol=0, atol=1e-15)


def _visible_v_mean(case, t, h, topk_row):
    r, loc = divmod(t, case.dql)
    pos = int(case.seq_lens[r]) - case.dql + loc
    rows = []
    for b in topk_row:
        if b < 0 or b * 128 > pos:
            continue
        n = min(128, pos - b * 128 + 1)
        p = case.block_table[r, b]
        rows.append(torch_values(case.kv[p, h, :n, 128:], case.kv_dtype).numpy())
    return np.concatenate(rows).mean(axis=0)


def test_identical_keys_give_mean_of_v():
    case = small_dense_case(8, 2, 3)
    kv = case.kv.copy()
    kv[..., :128] = 0x30  # every key row identical (0.5 in every entry)
    case.kv = kv
    out = run_oracle(case)
    g = case.num_q_heads // case.num_kv_heads
    for t in range(case.real_rows):
        for j in range(case.num_q_heads):
            ref = _visible_v_mean(case, t, j // g, case.topk[t, j // g])
            assert np.allclose(out[t, j], ref, rtol=0, atol=1e-12)


def test_zero_scale_gives_mean_of_v():
    case = small_dense_case(16, 1, 2)
    out = run_oracle(case, sm_scale=0.0)
    for t in range(case.real_rows):
        ref = _visible_v_mean(case, t, 0, case.topk[t, 0])
        assert np.allclose(out[t], ref[None, :], rtol=0, atol=1e-12)


def test_large_scale_picks_argmax_key():
    case = small_dense_case(8, 2, 1, pattern=(200, 300))
    scale = 1e4
    out = run_oracle(case, sm_scale=scale)
    vals = torch_values(case.kv, case.kv_dtype).numpy()
    q = torch_q(case.q, case.q_dtype, case.q_scale).numpy()
    g = case.num_q_heads // case.num_kv_heads
    checked = 0
    for t in range(case.real_rows):
        r = t // case.dql
        s = int(case.seq_lens[r])
        pages = case.block_table[r, :gen.pages_for(s)]
        for j in range(case.num_q_heads):
            h = j // g
            seqkv = vals[pages, h].reshape(-1, 256)[:s]
            logits = seqkv[:, :128] @ q[t, j]
            order = np.argsort(-logits)
            if (logits[order[0]] - logits[order[1]]) * scale < 60:
                continue
            assert np.allclose(out[t, j], seqkv[order[0], 128:], rtol=0, atol=1e-12)
            checked += 1
    assert checked > case.real_rows * case.num_q_heads // 2


# ---------------------------------------------------------------------------
# invariances and -1 handling
# ---------------------------------------------------------------------------

def _rand_case(**kw):
    base = dict(seed=11, batch=3, dql=3, num_q_heads=8, num_kv_heads=2, topk_k=6,
                seq_lo=300, seq_hi=1400)
    base.update(kw)
    return gen.make_random_case(**base)


def test_topk_row_order_invariance():
    case = _rand_case()
    a = run_oracle(case)
    rng = np.random.default_rng(0)
    perm = case.topk.copy()
    for t in range(perm.shape[0]):
        for h in range(perm.shape[1]):
            perm[t, h] = rng.permutation(perm[t, h])
    b = run_oracle(case, topk=perm)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_inserting_minus_one_changes_nothing():
    case = _rand_case()
    a = run_oracle(case)
    k = case.topk.shape[2]
    wide = np.full((case.topk.shape[0], case.topk.shape[1], 2 * k), -1, np.int32)
    rng = np.random.default_rng(1)
    for t in range(wide.shape[0]):
        for h in range(wide.shape[1]):
            slots = np.sort(rng.choice(2 * k, size=k, replace=False))
            wide[t, h, slots] = case.topk[t, h]
    b = run_oracle(case, topk=wide)
    assert np.array_equal(a, b)


def test_physical_page_relabelling_invariance():
    case = _rand_case()
    a = run_oracle(case)
    rng = np.random.default_rng(2)
    perm = rng.permutation(case.num_blocks)
    kv2 = np.empty_like(case.kv)
    kv2[perm] = case.kv
    bt2 = perm[case.block_table].astype(np.int32)
    b = run_oracle(case, kv=kv2, block_table=bt2)
    assert np.array_equal(a, b)


def test_poison_outside_visible_rows_changes_nothing():
    case = _rand_case()
    clean = gen.make_random_case(seed=11, batch=3, dql=3, num_q_heads=8, num_kv_heads=2,
                                 topk_k=6, seq_lo=300, seq_hi=1400, poison=False)
    a = run_oracle(clean)
    b = run_oracle(case)   # same draws, with NaN in tails and in the spare page
    assert not np.isnan(b).any()
    assert np.array_equal(a, b)


def test_invisible_indices_change_nothing():
    case = _rand_case(dql=4)
    a = run_oracle(case)
    k = case.topk.shape[2]
    extra = np.concatenate([case.topk, np.full(case.topk.shape[:2] + (2,), -1, np.int32)],
                           axis=2)
    for t in range(case.real_rows):
        r, loc = divmod(t, case.dql)
        pos = int(case.seq_lens[r]) - case.dql + loc
        extra[t, :, k] = pos // 128 + 1          # starts after pos
        extra[t, :, k + 1] = pos // 128 + 40     # far beyond the table row
    b = run_oracle(case, topk=extra)
    assert np.array_equal(a, b)


def _bad_table(case, seed):
    """The block table with about a third of each request's used entries
    naming no page of the pool (-1, num_blocks, num_blocks + 1000); returns
    it with the (request, block) pairs it spoiled."""
    rng = np.random.default_rng(seed)
    bt = case.block_table.copy()
    nb = case.kv.shape[0]
    spoiled = set()
    for r, s in enumerate(case.seq_lens):
        used = gen.pages_for(int(s))
        for b in rng.choice(used, size=max(1, used // 3), replace=False):
            bt[r, b] = rng.choice([-1, nb, nb + 1000])
            spoiled.add((r, int(b)))
    return bt, spoiled


def test_out_of_pool_table_entries_change_nothing_but_their_block():
    """A selected block whose table entry is no page of the pool contributes
    nothing: the same as a -1 in its place."""
    case = _rand_case(dql=2)
    bt, spoiled = _bad_table(case, 5)
    masked = case.topk.copy()
    for t in range(case.real_rows):
        r = t // case.dql
        for h in range(masked.shape[1]):
            for j in range(masked.shape[2]):
                if (r, int(masked[t, h, j])) in spoiled:
                    masked[t, h, j] = -1
    assert (masked != case.topk).any()
    a = run_oracle(case, block_table=bt)
    b = run_oracle(case, topk=masked)
    assert np.array_equal(a, b)


def test_scorer_out_of_pool_table_entries_score_minus_inf():
    case = _rand_case(dql=2)
    bt, spoiled = _bad_table(case, 6)
    good = run_scores(case)
    bad = run_scores(case, block_table=bt)
    for i in range(case.real_rows):
        r = i // case.dql
        for b in range(good.shape[1]):
            if (r, b) in spoiled:
                assert np.all(bad[:, b, i] == -np.inf)
            else:
                assert np.array_equal(bad[:, b, i], good[:, b, i])


def test_all_minus_one_and_padding_rows_are_zero():
    case = _rand_case(pad_rows=3)
    topk = case.topk.copy()
    topk[1] = -1
    out = run_oracle(case, topk=topk)
    assert np.all(out[1] == 0.0)
    assert np.all(out[case.real_rows:] == 0.0)
    assert np.all(np.abs(out[0]) > 0)


def test_row_subset_matches_full():
    case = _rand_case()
    full = run_oracle(case)
    sub = run_oracle(case, rows=[5, 2])
    assert np.array_equal(sub, full[[5, 2]])


# ---------------------------------------------------------------------------
# scorer
# ---------------------------------------------------------------------------

def brute_scores(case, max_blocks):
    """Triple loop over (h, b, t) and every (g, j) pair, torch-decoded K."""
    vals = torch_values(case.kv, case.kv_dtype).numpy()
    q = torch_q(case.q, case.q_dtype, case.q_scale).numpy()
    g = case.num_q_heads // case.num_kv_heads
    out = np.full((case.num_kv_heads, max_blocks, case.real_rows), -np.inf)
    for t in range(case.real_rows):
        r, loc = divmod(t, case.dql)
        pos = int(case.seq_lens[r]) - case.dql + loc
        for h in range(case.num_kv_heads):
            for b in range(max_blocks):
                best = -np.inf
                for key in range(b * 128, min(b * 128 + 128, pos + 1)):
                    p = case.block_table[r, key // 128]
                    krow = vals[p, h, key % 128, :128] * case.k_scale
                    for gg in range(g):
                        best = max(best, float(np.dot(q[t, h * g + gg], krow)))
                out[h, b, t] = best
    return out


def run_scores(case, max_blocks=None, **over):
    kw = dict(q_bits=case.q, kv=case.kv, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
              block_table=case.block_table, seq_lens=case.seq_lens,
              decode_query_len=case.dql, num_kv_heads=case.num_kv_heads,
              max_blocks=max_blocks or case.max_blocks, q_dtype=case.q_dtype,
              q_scale=case.q_scale)
    kw.update(over)
    return om.block_max_scores(**kw)


@pytest.mark.parametrize("kv_dtype,q_dtype,q_scale", [
    (gen.KV_FP8, gen.Q_BF16, 1.0), (gen.KV_BF16, gen.Q_BF16, 1.0),
    (gen.KV_E5M2, gen.Q_BF16, 1.0), (gen.KV_FP8, gen.Q_FP8, 0.5)])
def test_scorer_brute_force(kv_dtype, q_dtype, q_scale):
    case = gen.make_random_case(seed=21, batch=2, dql=2, num_q_heads=4, num_kv_heads=2,
                                topk_k=4, seq_lo=129, seq_hi=400, kv_dtype=kv_dtype,
                                q_dtype=q_dtype, q_scale=q_scale)
    case.k_scale = 0.5
    mb = case.max_blocks + 1
    a = run_scores(case, mb)
    b = brute_scores(case, mb)
    assert np.array_equal(np.isinf(a), np.isinf(b))
    fin = np.isfinite(b)
    assert np.allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


def test_scorer_one_hot_query():
    case = gen.make_random_case(seed=22, batch=2, dql=1, num_q_heads=4, num_kv_heads=1,
                                topk_k=4, seq_lo=200, seq_hi=600)
    d = 37
    q = np.zeros_like(case.q)
    q[..., d] = gen.encode_bf16(np.array([1.0]))[0]
    case.q = q
    sc = run_scores(case)
    vals = torch_values(case.kv, case.kv_dtype).numpy()
    for t in range(case.real_rows):
        pos = int(case.seq_lens[t]) - 1
        for b in range(case.max_blocks):
            if b * 128 > pos:
                assert sc[0, b, t] == -np.inf
                continue
            n = min(128, pos - b * 128 + 1)
            p = case.block_table[t, b]
            assert sc[0, b, t] == vals[p, 0, :n, d].max()


def test_scorer_zero_keys():
    case = gen.make_random_case(seed=23, batch=2, dql=2, num_q_heads=4, num_kv_heads=2,
                                topk_k=4, seq_lo=200, seq_hi=600, poison=False)
    kv = case.kv.copy()
    kv[..., :128] = 0
    case.kv = kv
    sc = run_scores(case)
    for t in range(case.real_rows):
        r, loc = divmod(t, case.dql)
        pos = int(case.seq_lens[r]) - case.dql + loc
        nvis = pos // 128 + 1
        assert np.all(sc[:, :nvis, t] == 0.0)
        assert np.all(sc[:, nvis:, t] == -np.inf)


# ---------------------------------------------------------------------------
# selector
# ---------------------------------------------------------------------------

def brute_topk(scores_1d, k):
    remaining = [b for b in range(len(scores_1d)) if scores_1d[b] > -math.inf]
    out = []
    while remaining and len(out) < k:
        best = remaining[0]
        for b in remaining[1:]:
            if scores_1d[b] > scores_1d[best]:
                best = b   # strict: the earlier (lower) index wins ties
        out.append(best)
        remaining.remove(best)
    return out + [-1] * (k - len(out))


def test_select_topk_golden_example():
    g = golden()["select_topk_example"]
    s = np.array([float(x) for x in g["scores"]])[None, :, None]
    got = om.select_topk(s, g["k"])
    assert got[0, 0].tolist() == g["expected"]


@pytest.mark.parametrize("tie_frac", [0.0, 0.3])
def test_select_topk_brute_force(tie_frac):
    seq = np.array([129, 700, 2000], dtype=np.int32)
    sc = gen.make_scores(31, 2, 16, 6, seq, 2, tie_frac=tie_frac)
    got = om.select_topk(sc, 5)
    for h in range(2):
        for t in range(6):
            assert got[t, h].tolist() == brute_topk(sc[h, :, t].astype(np.float64), 5)


def test_select_topk_pads_when_few_visible():
    s = np.full((1, 8, 1), -np.inf)
    s[0, 2, 0] = 1.0
    s[0, 5, 0] = 1.0
    assert om.select_topk(s, 4)[0, 0].tolist() == [2, 5, -1, -1]


# ---------------------------------------------------------------------------
# the 4-bit (MXFP4 head-slot) cache
# ---------------------------------------------------------------------------

# OCP Microscaling Formats (MX) v1.0 specification, FP4 (E2M1) element
# encoding: the 16 codes' values (sign bit 3).
OCP_E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                   -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_matches_ocp_table():
    got = om.decode_e2m1(np.arange(16))
    assert np.array_equal(got, np.array(OCP_E2M1_VALUES))
    assert np.array_equal(np.signbit(got), np.signbit(np.array(OCP_E2M1_VALUES)))
    # only the low nibble is a code
    assert np.array_equal(om.decode_e2m1(np.arange(16) + 0xA0), got)


def test_e8m0_decode_exhaustive_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64)
    got = om.decode_e8m0(np.arange(256))
    assert np.array_equal(np.isnan(got), torch.isnan(ref).numpy())
    fin = ~np.isnan(got)
    assert np.array_equal(got[fin], ref.numpy()[fin])
    assert got[127] == 1.0 and np.isnan(got[255])


def test_mxfp4_head_slots_tile_each_head_run():
    """As the test page's head-slot test: slot 2h (K) and 2h+1 (V) hold head
    h's data then scales, so each head is one contiguous run of the page."""
    hkv = 4
    rng = np.random.default_rng(5)
    kv = rng.integers(0, 256, size=(3, 2 * hkv, 128, 68), dtype=np.uint8)
    runs = kv.reshape(3, hkv, 2 * om.MXFP4_SLOT_BYTES)
    assert om.MXFP4_SLOT_BYTES == 128 * (128 // 2 + 128 // 32)
    for p in range(3):
        for h in range(hkv):
            parts = []
            for side in (0, 1):
                data, scales = om.mxfp4_slot(kv, p, h, side)
                assert data.shape == (128, 64) and scales.shape == (128, 4)
                parts += [data.reshape(-1), scales.reshape(-1)]
            assert np.array_equal(np.concatenate(parts), runs[p, h])


def fp4_values(rng, shape):
    """Values an MXFP4 block holds exactly: e2m1 grid values times 2^k per
    32-block, with one +-6 per block so the block scale is exactly 2^k."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = mags[rng.integers(0, 8, size=shape)] * rng.choice([-1.0, 1.0], size=shape)
    blocks = vals.reshape(shape[:-1] + (shape[-1] // 32, 32))
    lead = blocks.shape[:-1]
    at = rng.integers(0, 32, size=lead)
    np.put_along_axis(blocks, at[..., None],
                      (6.0 * rng.choice([-1.0, 1.0], size=lead))[..., None], axis=-1)
    blocks *= np.exp2(rng.integers(-6, 4, size=lead))[..., None]
    return blocks.reshape(shape)


def test_mxfp4_pack_round_trip_is_exact():
    rng = np.random.default_rng(6)
    x = fp4_values(rng, (3, 2, 128, 256))
    kv = gen.pack_mxfp4_pages(x)
    assert kv.shape == (3, 4, 128, 68)
    for p in range(3):
        for h in range(2):
            k, v = om.page_kv(kv, "mxfp4", 0.5, 2.0, p, h, 128)
            assert np.array_equal(k, x[p, h, :, :128] * 0.5)
            assert np.array_equal(v, x[p, h, :, 128:] * 2.0)
            k7, _ = om.page_kv(kv, "mxfp4", 1.0, 1.0, p, h, 7)
            assert np.array_equal(k7, x[p, h, :7, :128])


def small_fp4_case(hq=8, hkv=2, dql=2, pattern=(257, 513), seed=0, q_dtype=gen.Q_BF16,
                   q_scale=1.0, k_scale=0.5, v_scale=2.0):
    """A p3-shaped case whose 4-bit pool is packed from known values (returned
    beside the case), with NaN poison past seq_len and on the spare page."""
    case = gen.make_p3_case(hq, hkv, 1, dql, seq_pattern=pattern, seed=seed,
                            kv_dtype=gen.KV_MXFP4, topk_k=8, q_dtype=q_dtype,
                            q_scale=q_scale, k_scale=k_scale, v_scale=v_scale)
    rng = np.random.default_rng(77 + seed)
    vals = fp4_values(rng, (case.num_blocks, hkv, 128, 256))
    case.kv = gen.pack_mxfp4_pages(vals)
    used = set(int(x) for r, s in enumerate(case.seq_lens)
               for x in case.block_table[r, :gen.pages_for(s)])
    gen.fill_pages(case.kv, [p for p in range(case.num_blocks) if p not in used], gen.KV_MXFP4)
    gen.poison_tail_slots(case.kv, case.block_table, case.seq_lens, gen.KV_MXFP4)
    return case, vals


def fp4_pin_error(case, vals) -> float:
    return float(np.max(np.abs(run_oracle(case) - dense_reference(case, vals))))


@pytest.mark.parametrize("dql", [1, 4])
@pytest.mark.parametrize("heads", [(8, 2), (16, 1)])
@pytest.mark.parametrize("qfmt", [(gen.Q_BF16, 1.0), (gen.Q_FP8, 0.5)])
def test_mxfp4_dense_equivalence(dql, heads, qfmt):
    case, vals = small_fp4_case(heads[0], heads[1], dql, q_dtype=qfmt[0], q_scale=qfmt[1])
    assert fp4_pin_error(case, vals) < 1e-12


def test_mxfp4_poisoned_pool_has_nan_scales_past_seq_len():
    case, _ = small_fp4_case()
    r, s = 0, int(case.seq_lens[0])
    page = case.block_table[r, gen.pages_for(s) - 1]
    used = s - (gen.pages_for(s) - 1) * 128
    _, scales = om.mxfp4_slot(case.kv, page, 0, 1)
    assert np.isnan(om.decode_e8m0(scales[used:])).all()
    assert not np.isnan(om.decode_e8m0(scales[:used])).any()


def test_mxfp4_scorer_brute_force():
    case, vals = small_fp4_case(8, 2, 2, pattern=(300, 700))
    mb = int(case.block_table.shape[1])
    got = om.block_max_scores(case.q, case.kv, case.kv_dtype, case.k_scale, case.block_table,
                              case.seq_lens, case.dql, case.num_kv_heads, mb)
    q = torch_q(case.q).numpy()
    g = case.num_q_heads // case.num_kv_heads
    for t in range(case.real_rows):
        r, loc = divmod(t, case.dql)
        pos = int(case.seq_lens[r]) - case.dql + loc
        for h in range(case.num_kv_heads):
            for b in range(mb):
                if b * 128 > pos:
                    assert got[h, b, t] == -np.inf
                    continue
                n = min(128, pos - b * 128 + 1)
                k = vals[case.block_table[r, b], h, :n, :128] * case.k_scale
                want = max(float(np.dot(q[t, h * g + j], k[i])) for j in range(g)
                           for i in range(n))
                assert abs(got[h, b, t] - want) <= 1e-12 * max(1.0, abs(want))


# ---------------------------------------------------------------------------
# planted mistakes: each must trip at least one pin
# ---------------------------------------------------------------------------

_mxfp4_slot = om.mxfp4_slot
_page_kv = om.page_kv


def _rows_high_nibble_first(data, scales, n):
    d = np.arange(128)
    code = (data[:n, d // 2].astype(np.int64) >> (4 * (1 - d % 2))) & 0xF
    return om.decode_e2m1(code) * om.decode_e8m0(scales[:n, d // 32])


def _rows_scale_by_byte_block(data, scales, n):
    d = np.arange(128)
    code = (data[:n, d // 2].astype(np.int64) >> (4 * (d % 2))) & 0xF
    return om.decode_e2m1(code) * om.decode_e8m0(scales[:n, (d // 2) // 32])


def _slot_writer_order(kv, page, head, side):
    """The writer's order (every head's slot of one side, then the other)."""
    hkv = kv.shape[1] // 2
    flat = np.asarray(kv[int(page), side * hkv + int(head)]).reshape(-1)
    return (flat[:om.MXFP4_DATA_BYTES].reshape(128, 64),
            flat[om.MXFP4_DATA_BYTES:].reshape(128, 4))


def _e2m1_bias_0(codes):
    """e2m1 read with exponent bias 0 instead of 1."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    e, m = (c >> 1) & 3, c & 1
    sign = np.where((c >> 3) & 1 == 1, -1.0, 1.0)
    return sign * np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e.astype(float)))


def _page_kv_no_global_scale(kv, kv_dtype, k_scale, v_scale, page, head, n):
    if kv_dtype == "mxfp4":
        return _page_kv(kv, kv_dtype, 1.0, 1.0, page, head, n)
    return _page_kv(kv, kv_dtype, k_scale, v_scale, page, head, n)


FP4_MUTANTS = {
    "fp4_high_nibble_first": ("mxfp4_rows", _rows_high_nibble_first),
    "fp4_scale_block_of_byte": ("mxfp4_rows", _rows_scale_by_byte_block),
    "fp4_kv_slots_swapped": ("mxfp4_slot",
                             lambda kv, page, head, side: _mxfp4_slot(kv, page, head, 1 - side)),
    "fp4_writer_slot_order": ("mxfp4_slot", _slot_writer_order),
    "e8m0_bias_128": ("decode_e8m0", lambda c: np.where(np.asarray(c) == 255, np.nan,
                                                        np.exp2(np.asarray(c, float) - 128))),
    "e2m1_bias_0": ("decode_e2m1", _e2m1_bias_0),
    "fp4_global_scale_ignored": ("page_kv", _page_kv_no_global_scale),
}

MUTANTS = {
    "visible_rows_off_by_one": ("visible_rows",
                                lambda pos, b: 0 if b < 0 or b * 128 > pos
                                else min(128, pos - b * 128)),
    "causal_start_strict": ("visible_rows",
                            lambda pos, b: 0 if b < 0 or b * 128 >= pos
                            else min(128, pos - b * 128 + 1)),
    "position_plus_one": ("token_position", lambda s, dql, loc: int(s) - int(dql) + int(loc) + 1),
    "kv_head_modulo": ("kv_head_of", lambda j, g: j % 2),
    "kv_swapped": ("split_kv", lambda raw: (raw[:, 128:], raw[:, :128])),
    "no_sm_scale": ("softmax_attend",
                    lambda qv, k, v, sc: (lambda z: (np.exp(z - z.max()) @ v)
                                          / np.exp(z - z.max()).sum())(k @ qv)),
    "scale_ignored": ("dequant", lambda raw, dt, scale: (
        om._E4M3_TABLE[np.asarray(raw, dtype=np.uint8)] if dt == "fp8_e4m3"
        else om._E5M2_TABLE[np.asarray(raw, dtype=np.uint8)] if dt == "fp8_e5m2"
        else om.decode_bf16(raw))),
    "q_scale_ignored": ("decode_query", lambda q, dt, scale: (
        om._E4M3_TABLE[np.asarray(q, dtype=np.uint8)] if dt == "fp8_e4m3"
        else om.decode_bf16(q))),
    "e5m2_bias_16": ("dequant", lambda raw, dt, scale: (
        om.decode_e5m2(raw) * 0.5 * scale if dt == "fp8_e5m2"
        else om._E4M3_TABLE[np.asarray(raw, dtype=np.uint8)] * scale if dt == "fp8_e4m3"
        else om.decode_bf16(raw) * scale)),
}


def _pins_pass():
    cases = [small_dense_case(8, 2, 4), small_dense_case(8, 2, 1),
             small_dense_case(8, 2, 3, k_scale=0.5, v_scale=2.0),
             small_dense_case(8, 2, 2, gen.KV_E5M2, q_dtype=gen.Q_FP8, q_scale=0.5)]
    if not all(dense_pin_error(c) < 1e-12 for c in cases):
        return False
    case, vals = small_fp4_case(8, 2, 2)
    return fp4_pin_error(case, vals) < 1e-12


def test_pins_pass_on_clean_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(FP4_MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name] if name in MUTANTS else FP4_MUTANTS[name]
    monkeypatch.setattr(om, attr, fn)
    try:
        ok = _pins_pass()
    except (AssertionError, IndexError, ValueError):
        ok = False
    assert not ok, f"planted mistake {name} was not caught"


def test_planted_scorer_mistakes_are_caught(monkeypatch):
    case = gen.make_random_case(seed=24, batch=2, dql=2, num_q_heads=4, num_kv_heads=2,
                                topk_k=4, seq_lo=129, seq_hi=400)
    ref = brute_scores(case, case.max_blocks)
    monkeypatch.setattr(om, "visible_rows",
                        lambda pos, b: 0 if b < 0 or b * 128 > pos else 128)
    with np.errstate(invalid="ignore"):
        bad = run_scores(case)
    assert not np.array_equal(np.nan_to_num(bad), np.nan_to_num(ref))


def test_planted_selector_mistake_is_caught():
    g = golden()["select_topk_example"]
    s = np.array([float(x) for x in g["scores"]])
    # reversed tie rule: higher block id first among equal scores
    cand = [b for b in range(len(s)) if s[b] > -math.inf]
    cand.sort(key=lambda b: (-s[b], -b))
    assert cand[: g["k"]] != g["expected"]


# ---------------------------------------------------------------------------
# prefill (ragged query chunks over a cached context)
# ---------------------------------------------------------------------------

def dense_prefill_reference(case: gen.PrefillCase) -> np.ndarray:
    """Causal GQA attention of each request's prefill chunk over its whole
    un-paged sequence via SDPA in float64: local token i sees keys 0..ctx+i."""
    hq, hkv = case.num_q_heads, case.num_kv_heads
    g = hq // hkv
    vals = torch_values(case.kv, case.kv_dtype)
    q = torch_q(case.q, case.q_dtype, case.q_scale)
    out = torch.zeros(case.num_token_rows, hq, 128, dtype=torch.float64)
    for r in range(case.batch):
        s, ql, c0 = int(case.seq_lens[r]), int(case.q_lens[r]), int(case.cu_seqlens_q[r])
        if ql == 0:
            continue
        n = gen.pages_for(s)
        pages = torch.from_numpy(case.block_table[r, :n].astype(np.int64))
        seqkv = vals[pages].permute(1, 0, 2, 3).reshape(hkv, n * 128, 256)[:, :s]
        k = (seqkv[..., :128] * case.k_scale).repeat_interleave(g, dim=0)
        v = (seqkv[..., 128:] * case.v_scale).repeat_interleave(g, dim=0)
        qh = q[c0:c0 + ql].permute(1, 0, 2)
        pos = int(case.context_lens[r]) + torch.arange(ql)
        mask = torch.arange(s)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qh, k, v, attn_mask=mask, scale=case.sm_scale)
        out[c0:c0 + ql] = o.permute(1, 0, 2)
    return out.numpy()


def run_prefill_oracle(case: gen.PrefillCase, **over):
    kw = dict(q_bits=case.q, kv=case.kv, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
              v_scale=case.v_scale, block_table=case.block_table,
              cu_seqlens_q=case.cu_seqlens_q, context_lens=case.context_lens, topk=case.topk,
              num_kv_heads=case.num_kv_heads, sm_scale=case.sm_scale, q_dtype=case.q_dtype,
              q_scale=case.q_scale)
    kw.update(over)
    return om.sparse_prefill(**kw)


def _prefill_pin_error(case):
    return float(np.max(np.abs(run_prefill_oracle(case) - dense_prefill_reference(case))))


@pytest.mark.parametrize("heads", [(8, 2), (16, 1)])
@pytest.mark.parametrize("fmt", [(gen.KV_FP8, gen.Q_BF16, 1.0), (gen.KV_FP8, gen.Q_FP8, 0.5),
                                 (gen.KV_BF16, gen.Q_BF16, 1.0)])
def test_prefill_dense_equivalence_test_page_shape(heads, fmt):
    """The test page's prefill shape: q_lens (300, 128, 77) over seq_lens
    (300, 640, 1100), every causally visible page selected."""
    kv_dtype, q_dtype, q_scale = fmt
    case = gen.make_prefill_case(31, [300, 128, 77], [300, 640, 1100], heads[0], heads[1],
                                 kv_dtype=kv_dtype, q_dtype=q_dtype, q_scale=q_scale)
    case.k_scale, case.v_scale = 0.5, 2.0
    assert _prefill_pin_error(case) < 1e-12


def test_prefill_chunks_with_empty_request_and_padding():
    case = gen.make_prefill_case(32, [5, 0, 64, 1], [700, 300, 129, 1], 8, 2, pad_rows=3)
    assert _prefill_pin_error(case) < 1e-12
    out = run_prefill_oracle(case)
    assert np.all(out[case.real_rows:] == 0.0)
    assert om.prefill_request_of(case.cu_seqlens_q, 5) == 2      # request 1 owns no row


def test_prefill_with_uniform_chunks_is_decode():
    """cu = r*dql and context = seq - dql make the prefill definition the
    decode one: the two functions agree exactly."""
    dcase = gen.make_random_case(seed=33, batch=3, dql=3, num_q_heads=8, num_kv_heads=2,
                                 topk_k=8, seq_lo=129, seq_hi=900, pad_rows=2)
    cu = np.arange(dcase.batch + 1, dtype=np.int32) * dcase.dql
    ctx = dcase.seq_lens - dcase.dql
    a = run_oracle(dcase)
    b = om.sparse_prefill(dcase.q, dcase.kv, dcase.kv_dtype, dcase.k_scale, dcase.v_scale,
                          dcase.block_table, cu, ctx, dcase.topk, dcase.num_kv_heads,
                          dcase.sm_scale)
    assert np.array_equal(a, b)


def test_planted_prefill_mistakes_are_caught(monkeypatch):
    case = gen.make_prefill_case(34, [40, 9], [300, 200], 8, 2)
    assert _prefill_pin_error(case) < 1e-12
    monkeypatch.setattr(om, "prefill_position", lambda c, s, t: int(c) + int(t) - int(s) + 1)
    with np.errstate(invalid="ignore"):
        assert not _prefill_pin_error(case) < 1e-12
    monkeypatch.undo()
    real = om.prefill_request_of
    monkeypatch.setattr(om, "prefill_request_of",
                        lambda cu, t: (lambda r: None if r is None else max(0, r - 1))(real(cu, t)))
    with np.errstate(invalid="ignore"):
        assert not _prefill_pin_error(case) < 1e-12



# ---------------------------------------------------------------------------
# dense decode (every visible block)
# ---------------------------------------------------------------------------

def run_dense_oracle(case, **over):
    kw = dict(q_bits=case.q, kv=case.kv, kv_dtype=case.kv_dtype, k_scale=case.k_scale,
              v_scale=case.v_scale, block_table=case.block_table, seq_lens=case.seq_lens,
              decode_query_len=case.dql, num_kv_heads=case.num_kv_heads,
              sm_scale=case.sm_scale, q_dtype=case.q_dtype, q_scale=case.q_scale)
    kw.update(over)
    return om.dense_decode(**kw)


@pytest.mark.parametrize("dql", [1, 4])
@pytest.mark.parametrize("fmt", [(gen.KV_FP8, gen.Q_BF16, 1.0), (gen.KV_E5M2, gen.Q_FP8, 0.5)])
def test_dense_decode_equals_sdpa(dql, fmt):
    """No top-k: causal attention over the whole un-paged sequence."""
    kv_dtype, q_dtype, q_scale = fmt
    case = small_dense_case(8, 2, dql, kv_dtype, pattern=(257, 1300), q_dtype=q_dtype,
                            q_scale=q_scale)
    got = run_dense_oracle(case)
    assert float(np.max(np.abs(got - dense_reference(case)))) < 1e-12


def test_dense_decode_planted_mistake_is_caught(monkeypatch):
    case = small_dense_case(8, 2, 3, pattern=(300, 700))
    monkeypatch.setattr(om, "visible_rows",
                        lambda pos, b: 0 if b < 0 or b * 128 > pos else min(128, pos - b * 128))
    assert not float(np.max(np.abs(run_dense_oracle(case) - dense_reference(case)))) < 1e-12


def test_dense_decode_rows_without_live_keys_are_zeros():
    """Rows that see no key -- a position before the first key (seq_len <
    decode_query_len), or every visible block outside the pool -- are exact
    zeros (the zero-row rule for padding and empty rows); every other row
    still equals causal SDPA over its request's sequence."""
    case = small_dense_case(8, 2, 4, pattern=(257, 513), pairs=2)
    case.seq_lens = case.seq_lens.copy()
    case.seq_lens[0] = 2                                   # positions -2, -1, 0, 1
    ref = dense_reference(case)                            # before the pool change
    case.block_table = case.block_table.copy()
    case.block_table[1, :] = case.kv.shape[0]              # no page of the pool
    got = run_dense_oracle(case)
    dql = case.dql
    empty = [0, 1] + list(range(dql, 2 * dql))             # request 0 rows 0-1, request 1
    assert np.all(got[empty] == 0.0)
    live = [t for t in range(case.batch * dql) if t not in empty]
    assert len(live) >= 2 * dql
    assert np.all(np.isfinite(ref[live]))
    assert float(np.max(np.abs(got[live] - ref[live]))) < 1e-12
