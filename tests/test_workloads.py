"""CPU checks of the seeded synthetic workloads (workloads/gen.py): that the
inputs have the structure their recipe states, so the parity tests and the
bench run on the workloads they claim.

* Paged layout over a shuffled physical pool with spare pages
  (``_make_paged_layout`` of the vLLM test file): every request owns
  ceil(seq/128) distinct pages, no page is owned twice, spare pages are owned
  by nobody.
* Index rows: distinct logical blocks inside the token's causal range,
  always including its own (last visible) block, -1 only as trailing padding
  (``_make_topk``; the always-include-last reading).
* Poison: rows past seq_len in each request's last page, and every spare
  page, hold NaN patterns (4-bit pages: NaN block scales); visible rows do not.
* Named-workload facts: c4's 8 long / 8 short requests and 4 padding rows;
  c5's log-normal sequence lengths; the prefill rules.
* The 4-bit encoder: the OCP MX block scale rule and the e2m1 rounding bound.
* Determinism: the same seed gives the same bytes.
"""
import math

import numpy as np
import pytest

import oracle.msa_oracle as om
from workloads import gen


@pytest.fixture(scope="module")
def c2():
    return gen.make_config("c2_tp4_fp8")


@pytest.fixture(scope="module")
def c4():
    return gen.make_config("c4_spec_ragged")


def _owned_pages(case):
    return [case.block_table[r, :gen.pages_for(s)] for r, s in enumerate(case.seq_lens)]


def _check_layout(case):
    owned = np.concatenate(_owned_pages(case))
    assert len(np.unique(owned)) == len(owned), "a physical page is owned twice"
    assert owned.min() >= 0 and owned.max() < case.num_blocks
    spare = np.setdiff1d(np.arange(case.num_blocks), owned)
    assert len(owned) + len(spare) == case.num_blocks
    return owned, spare


def _check_rows(topk_rows, positions, k, include_last=True):
    """topk_rows [T, Hkv, k] against positions [T]."""
    for t, pos in enumerate(positions):
        last = int(pos) // 128
        for row in topk_rows[t]:
            valid = row[row >= 0]
            n = len(valid)
            assert np.all(row[n:] == -1), "-1 only as trailing padding"
            assert len(np.unique(valid)) == n, "duplicate block in a row"
            assert np.all(valid <= last), "a block past the causal limit"
            if include_last:
                assert last in valid, "the token's own block is missing"
            assert n == min(k, last + 1)


def test_generation_is_deterministic():
    a = gen.make_config("c1_tiny_bf16", replicas=2)
    b = gen.make_config("c1_tiny_bf16", replicas=2)
    for x, y in [(a.kv, b.kv), (a.q, b.q), (a.topk, b.topk), (a.block_table, b.block_table)]:
        assert np.array_equal(x, y)
    for (qa, ta), (qb, tb) in zip(a.replicas, b.replicas):
        assert np.array_equal(qa, qb) and np.array_equal(ta, tb)
    r1 = gen.make_random_case(77, 3, 2, 16, 2, 8, 100, 2000, kv_dtype=gen.KV_MXFP4, k_scale=0.5)
    r2 = gen.make_random_case(77, 3, 2, 16, 2, 8, 100, 2000, kv_dtype=gen.KV_MXFP4, k_scale=0.5)
    assert np.array_equal(r1.kv, r2.kv) and np.array_equal(r1.topk, r2.topk)
    p1 = gen.make_prefill_case(5, [30, 0, 17], [300, 40, 500], 16, 2, rule="zipf")
    p2 = gen.make_prefill_case(5, [30, 0, 17], [300, 40, 500], 16, 2, rule="zipf")
    assert np.array_equal(p1.topk, p2.topk) and np.array_equal(p1.q, p2.q)


def test_pool_chunks_do_not_depend_on_pool_size():
    """Page chunk i of a pool comes from its own seed (pool seed, i), so it is
    the same whatever the pool's total size, and chunks differ."""
    big = gen.make_pool(np.random.default_rng(3), 600, 2, gen.KV_FP8, 0.5, chunk_pages=256)
    small = gen.make_pool(np.random.default_rng(3), 300, 2, gen.KV_FP8, 0.5, chunk_pages=256)
    assert np.array_equal(big[:256], small[:256])
    assert not np.array_equal(big[:44], big[256:300])
    assert np.array_equal(big[256:300], small[256:300])


def test_c1_layout_rows_and_poison():
    c = gen.make_config("c1_tiny_bf16")
    owned, spare = _check_layout(c)
    assert c.num_blocks == 16 and len(spare) == 4
    _check_rows(c.topk, c.positions(), c.topk_k)
    vals = om.decode_bf16(c.kv)
    for p in spare:
        assert np.isnan(vals[p]).all()
    for r, s in enumerate(c.seq_lens):
        last_page = c.block_table[r, gen.pages_for(s) - 1]
        used = int(s) - (gen.pages_for(s) - 1) * 128
        assert np.isfinite(vals[last_page, :, :used]).all()
        assert np.isnan(vals[last_page, :, used:]).all()


def test_c2_layout_and_rows(c2):
    _check_layout(c2)
    assert c2.batch == 32 and c2.dql == 4 and c2.topk_k == 16
    assert np.all((c2.seq_lens >= 16384) & (c2.seq_lens <= 65536))
    _check_rows(c2.topk, c2.positions(), 16)
    # one list per token, shared by the (single) kv head
    assert c2.topk.shape == (128, 1, 16)
    for r, s in enumerate(c2.seq_lens):
        last_page = c2.block_table[r, gen.pages_for(s) - 1]
        used = int(s) - (gen.pages_for(s) - 1) * 128
        if used < 128:
            assert np.all(c2.kv[last_page, :, used:] == gen.FP8_NAN_CODE)
        assert not np.any(c2.kv[last_page, :, :used] == gen.FP8_NAN_CODE)


def test_c4_structure(c4):
    _check_layout(c4)
    long_r = np.nonzero(c4.seq_lens == 131072)[0]
    short_r = np.nonzero(c4.seq_lens < 131072)[0]
    assert len(long_r) == 8 and len(short_r) == 8
    assert np.all((c4.seq_lens[short_r] >= 200) & (c4.seq_lens[short_r] <= 1900))
    assert c4.num_token_rows == 516 and c4.real_rows == 512
    assert np.all(c4.topk[512:] == -1)
    pos = c4.positions()
    _check_rows(c4.topk[:512], pos, 16)
    for t in range(512):
        if t // 32 in short_r:
            # every visible block of a short request
            for row in c4.topk[t]:
                assert sorted(row[row >= 0].tolist()) == list(range(int(pos[t]) // 128 + 1))


def test_zipf_recent_rule_prefers_recent_blocks():
    rng = np.random.default_rng(0)
    last, k = 400, 16
    counts = np.zeros(last + 1)
    for _ in range(400):
        for b in gen.pick_zipf_recent(rng, last, k):
            counts[b] += 1
    assert counts[last] == 400
    near, far = counts[last - 8:last].sum(), counts[:8].sum()
    assert near > 5 * far
    # the Gumbel form of the same draw, per head
    heads = gen.pick_zipf_recent_heads(rng, last, k, 4)
    for row in heads:
        assert last in row and len(np.unique(row)) == k


def test_c5_sequence_lengths():
    s = gen.c5_seq_lens(np.random.default_rng(5), B=4096)
    assert s.min() >= 8192 and s.max() <= 262144
    logs = np.log(s.astype(np.float64))
    mu, sigma = math.log(math.sqrt(8192.0 * 262144.0)), math.log(32.0) / 4.0
    assert abs(np.median(logs) - mu) < 0.05
    # the clip sits at mu +- 2 sigma: the 16th..84th percentile spread (2 sigma)
    # is untouched, and about 2.3% of draws land on each bound
    q16, q84 = np.percentile(logs, [15.87, 84.13])
    assert abs((q84 - q16) - 2 * sigma) < 0.1
    assert 0.01 < np.mean(s == 8192) < 0.04 and 0.01 < np.mean(s == 262144) < 0.04


def test_prefill_rules():
    p = gen.make_prefill_case(9, [300, 128, 77], [300, 640, 1100], 16, 1, pad_rows=3)
    assert list(p.cu_seqlens_q) == [0, 300, 428, 505]
    assert list(p.context_lens) == [0, 512, 1023]
    pos = p.positions()
    assert np.all(p.topk[505:] == -1)
    for t in range(505):
        last = int(pos[t]) // 128
        assert p.topk[t, 0, :last + 1].tolist() == list(range(last + 1))   # every visible
        assert np.all(p.topk[t, 0, last + 1:] == -1)
    z = gen.make_prefill_case(9, [64, 32], [5000, 9000], 16, 2, rule="zipf")
    _check_rows(z.topk, z.positions(), 16)


def test_mxfp4_encoder_scale_rule_and_rounding():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(
        np.float32)
    data, scales = gen.encode_mxfp4(x)
    blocks = x.reshape(64, 4, 32)
    amax = np.abs(blocks).max(axis=-1)
    want = np.floor(np.log2(amax)).astype(np.int64) - 2 + 127
    assert np.array_equal(scales.astype(np.int64), want)
    dec = om.mxfp4_rows(data, scales, 64).reshape(64, 4, 32)
    s = np.exp2(want - 127.0)[..., None]
    y = np.abs(blocks) / s
    # half the e2m1 spacing below 6, and saturation at 6 above
    bound = np.where(y < 2, 0.25, np.where(y < 4, 0.5, np.where(y <= 6, 1.0, y - 6.0))) * s
    assert np.all(np.abs(blocks - dec) <= bound + 1e-12)
    assert np.all(np.abs(dec) <= 6 * s)


def test_mxfp4_pool_poison():
    c = gen.make_random_case(91, 3, 1, 16, 2, 8, 100, 1000, kv_dtype=gen.KV_MXFP4)
    owned, spare = _check_layout(c)
    for p in spare:
        for h in range(c.num_kv_heads):
            for side in (0, 1):
                _, sc = om.mxfp4_slot(c.kv, p, h, side)
                assert np.all(sc == 255)
    for r, s in enumerate(c.seq_lens):
        page = c.block_table[r, gen.pages_for(s) - 1]
        used = int(s) - (gen.pages_for(s) - 1) * 128
        for h in range(c.num_kv_heads):
            for side in (0, 1):
                _, sc = om.mxfp4_slot(c.kv, page, h, side)
                assert np.all(sc[used:] == 255) and np.all(sc[:used] != 255)
