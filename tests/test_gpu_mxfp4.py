"""GPU parity of the 4-bit (MXFP4 head-slot) KV cache against the float64
oracle.

The cache is the NVFP4 head-slot page of vLLM's MSA test file with OCP MX
blocks (e2m1 codes, one E8M0 scale per 32 head dims) and global k / v scales
0.5 / 2.0, as in that file's NVFP4 decode test.  Cases: the dequant entry point
bit-exact on every page; the test page's decode shapes (heads (64,4) and
(16,1), query lengths 1..8) with bf16 and fp8 q; randomized cases with
padding rows, -1 entries and every split count, on single-row and 2- and
4-row tiles; dense decode; the test page's prefill shape (q_lens 300/128/77
over seq_lens 300/640/1100) with an fp8 q.  Stale rows of every last page hold
NaN block scales and spare pages are all NaN scales, so a read of a
non-visible row shows in the output.  Tolerance as for the other formats.
"""
import numpy as np
import pytest
import torch

import block_sparse_gqa_decode_amd as msa
from oracle import msa_oracle as om
from workloads import gen

from gpu_helpers import (DevCase, PrefillDevCase, assert_parity, oracle_attend, oracle_dense,
                         oracle_prefill, to_f64)

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 0.5, 2.0


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def test_mxfp4_dequant_bit_exact():
    """msa_mxfp4_to_bf16 (the attend's own e2m1/E8M0 conversion) equals the
    oracle's decode on every row of every page, NaN scales included."""
    _banner("mxfp4 -> bf16, every page of a poisoned pool")
    case = gen.make_random_case(401, 3, 2, 16, 2, 8, 100, 1500, kv_dtype=gen.KV_MXFP4)
    kv = torch.from_numpy(case.kv).cuda()
    nb, hkv = case.num_blocks, case.num_kv_heads
    out = torch.empty(nb, hkv, 128, 256, dtype=torch.bfloat16, device="cuda")
    msa.msa_mxfp4_to_bf16(kv, out, num_kv_heads=hkv)
    torch.cuda.synchronize()
    got = to_f64(out)
    for p in range(nb):
        for h in range(hkv):
            ref = np.concatenate([om.mxfp4_rows(*om.mxfp4_slot(case.kv, p, h, side), 128)
                                  for side in (0, 1)], axis=1)
            assert np.array_equal(np.isnan(got[p, h]), np.isnan(ref))
            fin = ~np.isnan(ref)
            assert np.array_equal(got[p, h][fin], ref[fin]), (p, h)


def test_mxfp4_dequant_extreme_scales():
    """Block scales 2^-127 (code 0), 2^-126, 2^0, 2^126, 2^127 (code 254) and NaN
    (code 255) over every e2m1 code: the conversion is exact wherever the
    product is in bf16 range (bf16 keeps subnormals)."""
    _banner("mxfp4 -> bf16, extreme block scales")
    nb, hkv = 1, 1
    kv = np.zeros((nb, 2 * hkv, 128, 68), dtype=np.uint8)
    flat = kv.reshape(nb, 2 * hkv, -1)
    codes = np.arange(16, dtype=np.uint8)
    data = np.tile((codes[0::2] | (codes[1::2] << 4)), 8)          # 64 bytes per row
    flat[:, :, :om.MXFP4_DATA_BYTES] = np.tile(data, 128)
    scale_codes = np.array([0, 1, 127, 253, 254, 255, 100, 150], dtype=np.uint8)
    scales = np.resize(scale_codes, 128 * 4)
    flat[:, :, om.MXFP4_DATA_BYTES:] = scales
    out = torch.empty(nb, hkv, 128, 256, dtype=torch.bfloat16, device="cuda")
    msa.msa_mxfp4_to_bf16(torch.from_numpy(kv).cuda(), out, num_kv_heads=hkv)
    torch.cuda.synchronize()
    got = to_f64(out)[0, 0]
    ref = np.concatenate([om.mxfp4_rows(*om.mxfp4_slot(kv, 0, 0, side), 128)
                          for side in (0, 1)], axis=1)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    inrange = ~np.isnan(ref) & (np.abs(ref) <= bf16_max)
    assert np.array_equal(got[inrange], ref[inrange])
    over = ~np.isnan(ref) & (np.abs(ref) > bf16_max)
    assert over.any()
    # past the bf16 range: infinity or saturation, with the sign kept
    assert np.all(np.sign(got[over]) == np.sign(ref[over]))
    assert np.all(np.abs(got[over]) >= bf16_max)


P3 = [(64, 4, 4, 1), (64, 4, 4, 4), (64, 4, 2, 8), (16, 1, 8, 1), (16, 1, 16, 4)]


@pytest.mark.parametrize("hq,hkv,pairs,dql", P3)
@pytest.mark.parametrize("qfmt", [(gen.Q_BF16, 1.0), (gen.Q_FP8, 0.5)])
def test_mxfp4_p3_shapes(hq, hkv, pairs, dql, qfmt):
    _banner(f"mxfp4 p3 heads=({hq},{hkv}) pairs={pairs} dql={dql} q={qfmt}")
    case = gen.make_p3_case(hq, hkv, pairs, dql, seq_pattern=(257, 513), seed=3,
                            kv_dtype=gen.KV_MXFP4, q_dtype=qfmt[0], q_scale=qfmt[1],
                            k_scale=K_SCALE, v_scale=V_SCALE)
    d = DevCase(case)
    ref = oracle_attend(case)
    for splits in (0, 1, 3):
        out = d.new_out()
        d.run(d.plan(num_splits=splits), out=out)
        torch.cuda.synchronize()
        assert_parity(to_f64(out), ref, what=f"splits={splits}")


RANDOM = [
    # seed, batch, dql, hq, hkv, k, lo, hi, pad, neg, splits, tile_rows, q
    (411, 4, 4, 16, 1, 16, 2000, 20000, 2, 0.1, 2, 1, gen.Q_BF16),
    (412, 3, 2, 8, 2, 8, 1, 700, 3, 0.2, 1, 2, gen.Q_BF16),
    (413, 2, 8, 32, 4, 16, 129, 5000, 1, 0.0, 4, 4, gen.Q_FP8),
    (414, 5, 1, 64, 4, 16, 3000, 9000, 0, 0.3, 0, 1, gen.Q_FP8),
    (415, 2, 32, 16, 2, 16, 40, 4000, 4, 0.1, 2, 2, gen.Q_BF16),
    (416, 3, 3, 12, 3, 4, 200, 2000, 2, 0.0, 16, 4, gen.Q_BF16),
]


@pytest.mark.parametrize("seed,batch,dql,hq,hkv,k,lo,hi,pad,neg,splits,tile_rows,qd", RANDOM)
def test_mxfp4_random_cases(seed, batch, dql, hq, hkv, k, lo, hi, pad, neg, splits, tile_rows,
                            qd):
    _banner(f"mxfp4 random seed={seed} B={batch} dql={dql} heads=({hq},{hkv}) k={k} "
            f"splits={splits} tile={tile_rows} q={qd}")
    case = gen.make_random_case(seed, batch, dql, hq, hkv, k, lo, hi, kv_dtype=gen.KV_MXFP4,
                                pad_rows=pad, neg_frac=neg, q_dtype=qd,
                                q_scale=0.5 if qd == gen.Q_FP8 else 1.0, k_scale=K_SCALE,
                                v_scale=V_SCALE)
    d = DevCase(case)
    d.run(d.plan(num_splits=splits, tile_rows=tile_rows))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    assert_parity(got, oracle_attend(case), what=f"seed {seed}")
    if pad:
        assert np.all(got[case.real_rows:] == 0.0)


@pytest.mark.parametrize("dql,tile_rows,qd", [(1, 0, gen.Q_BF16), (4, 4, gen.Q_FP8),
                                              (2, 2, gen.Q_BF16)])
def test_mxfp4_dense_decode(dql, tile_rows, qd):
    _banner(f"mxfp4 dense decode dql={dql} tile={tile_rows} q={qd}")
    case = gen.make_random_case(421, 3, dql, 16, 2, 16, 300, 6000, kv_dtype=gen.KV_MXFP4,
                                pad_rows=2, q_dtype=qd, q_scale=0.5 if qd == gen.Q_FP8 else 1.0,
                                k_scale=K_SCALE, v_scale=V_SCALE)
    d = DevCase(case)
    d.run(d.plan(dense=True, tile_rows=tile_rows))
    torch.cuda.synchronize()
    assert_parity(to_f64(d.out), oracle_dense(case), what="dense")


@pytest.mark.parametrize("hq,hkv", [(64, 4), (16, 1)])
@pytest.mark.parametrize("tile_rows", [1, 2])
def test_mxfp4_prefill_test_page_shape(hq, hkv, tile_rows):
    """The test page's NVFP4 prefill test: q_lens 300/128/77 over seq_lens
    300/640/1100, every visible page, fp8 q; here on 4-bit head slots."""
    _banner(f"mxfp4 prefill heads=({hq},{hkv}) tile={tile_rows}")
    case = gen.make_prefill_case(431, [300, 128, 77], [300, 640, 1100], hq, hkv, topk_k=16,
                                 kv_dtype=gen.KV_MXFP4, q_dtype=gen.Q_FP8, q_scale=0.5,
                                 k_scale=K_SCALE, v_scale=V_SCALE, pad_rows=3)
    d = PrefillDevCase(case)
    d.run(d.plan(tile_rows=tile_rows))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted(set(rng.choice(case.num_token_rows, 96, replace=False).tolist())
                  | {0, 299, 300, 427, 428, 504, 505, 506, 507})
    got = to_f64(d.out)[rows]
    assert_parity(got, oracle_prefill(case, rows=rows), what="prefill rows")


def _extreme_scale_case(q_dtype, q_scale):
    """A 4-bit case whose visible rows carry E8M0 codes 0 and 255: request 0's
    first selected page of kv head 0 has K scale code 255 on row 0, request
    1's of kv head 1 has V scale code 255 on row 0, and request 2's of kv
    head 0 has K scale code 0 on rows 0..9 and V scale code 0 on rows
    10..19.  Returns the case and the oracle's output."""
    case = gen.make_random_case(431, 4, 2, 16, 2, 8, 2600, 4000, kv_dtype=gen.KV_MXFP4,
                                q_dtype=q_dtype, q_scale=q_scale, k_scale=K_SCALE,
                                v_scale=V_SCALE)
    case.kv = case.kv.copy()
    flat = case.kv.reshape(case.kv.shape[0], case.kv.shape[1], -1)
    base = om.MXFP4_DATA_BYTES

    def first_page(r, h):
        t = r * case.dql                         # the request's first token row
        b = int(case.topk[t, h, 0])
        assert b >= 0
        return int(case.block_table[r, b])

    flat[first_page(0, 0), 0, base + 4 * 0 + 1] = 255                 # K, head 0
    flat[first_page(1, 1), 2 * 1 + 1, base + 4 * 0 + 2] = 255         # V, head 1
    p2 = first_page(2, 0)
    flat[p2, 0, base:base + 4 * 10] = 0                               # K rows 0..9
    flat[p2, 1, base + 4 * 10:base + 4 * 20] = 0                      # V rows 10..19
    return case, oracle_attend(case)


@pytest.mark.parametrize("qd,qs", [(gen.Q_BF16, 1.0), (gen.Q_FP8, 0.5)])
@pytest.mark.parametrize("tile_rows", [1, 2])
def test_mxfp4_attend_extreme_scale_codes(qd, qs, tile_rows):
    """Where the attend widens 4-bit entries to bf16 it reads an E8M0 code as
    the fp32 pattern code << 23: code 0 counts as 0 instead of 2^-127 (a
    difference far below the tolerance) and code 255 (NaN) as +inf.  So rows
    whose visible keys carry code 0 match the oracle, and exactly the (row,
    q head) outputs that the oracle makes NaN (a visible K or V block scale
    of 255) come out non-finite."""
    _banner(f"mxfp4 attend with E8M0 codes 0 and 255 on visible rows, q={qd} "
            f"tile_rows={tile_rows}")
    case, ref = _extreme_scale_case(qd, qs)
    nan_ref = np.isnan(ref).any(axis=2)                 # [rows, Hq]
    assert nan_ref.any() and not nan_ref.all()
    d = DevCase(case)
    d.run(d.plan(tile_rows=tile_rows))
    torch.cuda.synchronize()
    got = to_f64(d.out)
    bad = ~np.isfinite(got).all(axis=2)
    diff = np.argwhere(bad != nan_ref)
    print(f"[parity] non-finite (row, q head): gpu {np.argwhere(bad).tolist()} "
          f"oracle {np.argwhere(nan_ref).tolist()} differ at {diff.tolist()}", flush=True)
    assert np.array_equal(bad, nan_ref)
    rows = [t for t in range(case.num_token_rows) if not nan_ref[t].any()]
    assert_parity(got[rows], ref[rows], what="extreme scale codes")
