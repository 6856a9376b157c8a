"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched).

* the built library loads and exports every function the header declares;
* argument validation runs before any HIP call and reports misuse with a
  status and a message -- the analogue of the static-dispatch and ValueError
  cases of the vLLM test file test_minimax_m3_msa_cutlass_sparse_decode.py
  (decode query length 1..32, page size 128, head size 128) and of
  MSACutlassDecodePlanCache.prepare's tensor checks.
"""
import ctypes
import glob
import os
import re

import pytest

import block_sparse_gqa_decode_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa_sparse_decode.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def header_functions(paths=None):
    """Every function the given headers (default: all of include/) declare."""
    names = []
    for path in (HEADERS if paths is None else paths):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:msa_status|const char\*|int32_t)\s+(msa_\w+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return msa.load_library()


def shape(**kw):
    base = dict(batch=32, decode_query_len=4, num_token_rows=0, page_table_stride=512,
                num_q_heads=16, num_kv_heads=1, page_size=128, head_dim=128, topk_blocks=16,
                kv_dtype=msa.KV_FP8_E4M3, num_splits=1, q_dtype=msa.Q_BF16, tile_rows=0)
    base.update(kw)
    return msa._Shape(*[base[f] for f, _ in msa._Shape._fields_])


def plan_status(lib, s, device=0):
    h = ctypes.c_void_p()
    st = lib.msa_sparse_decode_plan(ctypes.byref(s), device, ctypes.byref(h))
    if st == 0:
        lib.msa_sparse_decode_plan_destroy(h)
    return st, lib.msa_last_error().decode()


def test_header_declares_the_boundary():
    names = header_functions([HEADER])
    assert "msa_probe_read_runs" not in names          # a measurement aid, own header
    for required in ("msa_sparse_decode_plan", "msa_sparse_decode_run",
                     "msa_block_score_topk"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define MSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.msa_abi_version() == int(m.group(1))


def test_shape_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct msa_decode_shape \{(.*?)\} msa_decode_shape;", text,
                     flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"int32_t\s+([\w\s,]+);", body)
    names = [n.strip() for grp in fields for n in grp.split(",")]
    assert names == [f for f, _ in msa._Shape._fields_]


# The static-dispatch cases of the test page, as argument validation: query
# length 0 and 33 are rejected, 1..32 accepted.  Accepted shapes with one
# split make no HIP call, so they succeed here without a GPU.
@pytest.mark.parametrize("batch,dql,hq,hkv,ok", [
    (16, 4, 64, 4, True), (16, 4, 16, 1, True), (24, 4, 16, 1, True), (32, 4, 16, 1, True),
    (16, 1, 64, 4, True), (16, 1, 16, 1, True), (16, 2, 64, 4, True), (16, 2, 16, 1, True),
    (16, 32, 64, 4, True), (16, 0, 64, 4, False), (16, 33, 64, 4, False),
    (8, 4, 64, 4, True),   # no minimum batch here: that was a tile heuristic
])
def test_decode_query_len_bounds(lib, batch, dql, hq, hkv, ok):
    st, msg = plan_status(lib, shape(batch=batch, decode_query_len=dql, num_q_heads=hq,
                                     num_kv_heads=hkv))
    if ok:
        assert st == 0, msg
    else:
        assert st == msa.MSA_ERR_INVALID_ARG and "decode_query_len" in msg


@pytest.mark.parametrize("field,value,status,fragment", [
    ("page_size", 64, msa.MSA_ERR_UNSUPPORTED, "page_size"),
    ("head_dim", 64, msa.MSA_ERR_UNSUPPORTED, "head_dim"),
    ("num_kv_heads", 3, msa.MSA_ERR_INVALID_ARG, "multiple"),
    ("num_kv_heads", 0, msa.MSA_ERR_INVALID_ARG, "head counts"),
    ("num_q_heads", 64, msa.MSA_ERR_UNSUPPORTED, "GQA group"),
    ("topk_blocks", -1, msa.MSA_ERR_INVALID_ARG, "topk_blocks"),
    ("tile_rows", 3, msa.MSA_ERR_INVALID_ARG, "tile_rows"),
    ("tile_rows", 16, msa.MSA_ERR_INVALID_ARG, "tile_rows"),
    ("topk_blocks", 65, msa.MSA_ERR_UNSUPPORTED, "topk_blocks"),
    ("batch", 0, msa.MSA_ERR_INVALID_ARG, "batch"),
    ("page_table_stride", 0, msa.MSA_ERR_INVALID_ARG, "page_table_stride"),
    ("num_token_rows", 5, msa.MSA_ERR_INVALID_ARG, "num_token_rows"),
    ("kv_dtype", 7, msa.MSA_ERR_INVALID_ARG, "kv_dtype"),
    ("q_dtype", 2, msa.MSA_ERR_INVALID_ARG, "q_dtype"),
    ("num_splits", 17, msa.MSA_ERR_INVALID_ARG, "num_splits"),
    ("num_splits", -1, msa.MSA_ERR_INVALID_ARG, "num_splits"),
])
def test_plan_rejects_bad_shapes(lib, field, value, status, fragment):
    st, msg = plan_status(lib, shape(**{field: value}))
    assert st == status and fragment in msg, (st, msg)


@pytest.mark.parametrize("kv,q,ok", [
    (msa.KV_BF16, msa.Q_BF16, True), (msa.KV_FP8_E4M3, msa.Q_BF16, True),
    (msa.KV_FP8_E5M2, msa.Q_BF16, True), (msa.KV_FP8_E4M3, msa.Q_FP8_E4M3, True),
    (msa.KV_FP8_E5M2, msa.Q_FP8_E4M3, True), (msa.KV_BF16, msa.Q_FP8_E4M3, False),
    (msa.KV_MXFP4, msa.Q_BF16, True), (msa.KV_MXFP4, msa.Q_FP8_E4M3, True),
])
def test_plan_format_pairs(lib, kv, q, ok):
    """An fp8 q runs the fp8 x fp8 MFMA and needs an fp8 cache; every other
    pair is accepted."""
    st, msg = plan_status(lib, shape(kv_dtype=kv, q_dtype=q))
    if ok:
        assert st == 0, msg
    else:
        assert st == msa.MSA_ERR_UNSUPPORTED and "fp8 q" in msg


def test_plan_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.msa_sparse_decode_plan(None, 0, ctypes.byref(h)) == msa.MSA_ERR_INVALID_ARG
    s = shape()
    assert lib.msa_sparse_decode_plan(ctypes.byref(s), 0, None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_decode_plan(ctypes.byref(s), -1, ctypes.byref(h)) == \
        msa.MSA_ERR_INVALID_ARG


def test_binding_raises_value_error_subclass():
    with pytest.raises(msa.MsaInvalidArgument, match="decode_query_len"):
        msa.msa_sparse_decode_plan(16, 33, num_q_heads=64, num_kv_heads=4,
                                   page_table_stride=8, topk_blocks=16,
                                   kv_dtype=msa.KV_FP8_E4M3, num_splits=1, device=0)
    with pytest.raises(msa.MsaUnsupported, match="page_size"):
        msa.msa_sparse_decode_plan(16, 4, num_q_heads=64, num_kv_heads=4,
                                   page_table_stride=8, topk_blocks=16,
                                   kv_dtype=msa.KV_FP8_E4M3, num_splits=1, page_size=64,
                                   device=0)


def test_plan_info_reports_normalised_shape():
    plan = msa.msa_sparse_decode_plan(4, 3, num_q_heads=16, num_kv_heads=1,
                                      page_table_stride=10, topk_blocks=8,
                                      kv_dtype=msa.KV_BF16, num_splits=1, device=0)
    assert plan.num_token_rows == 12 and plan.num_splits == 1 and plan.arena_bytes == 0
    plan.close()


# ---------------------------------------------------------------------------
# run / score / select argument checks (all fail before any HIP call)
# ---------------------------------------------------------------------------

FAKE = 0x10000  # a 16-byte-aligned non-NULL address; never dereferenced here


def _plan(lib, **kw):
    h = ctypes.c_void_p()
    s = shape(**kw)
    assert lib.msa_sparse_decode_plan(ctypes.byref(s), 0, ctypes.byref(h)) == 0
    return h


def _run(lib, h, **over):
    args = dict(q=FAKE, kv=FAKE, kvs=(256 * 128, 256 * 128, 256, 1), nb=10, qs=1.0, ks=1.0,
                vs=1.0, bt=FAKE, sl=FAKE, tk=FAKE, tks=(16, 16, 1), out=FAKE, sm=0.088,
                stream=None)
    args.update(over)
    kvs = msa._I64x4(*args["kvs"]) if args["kvs"] is not None else None
    tks = msa._I64x3(*args["tks"]) if args["tks"] is not None else None
    st = lib.msa_sparse_decode_run(h, args["q"], args["kv"], kvs, args["nb"], args["qs"],
                                   args["ks"], args["vs"], args["bt"], args["sl"], args["tk"],
                                   tks, args["out"], args["sm"], args["stream"])
    return st, lib.msa_last_error().decode()


@pytest.mark.parametrize("over,fragment", [
    (dict(q=None), "q and out"),
    (dict(out=None), "q and out"),
    (dict(q=FAKE + 4), "aligned"),
    (dict(bt=None), "block_table"),
    (dict(tk=None), "block_table"),
    (dict(kv=None), "kv_cache is NULL"),
    (dict(kv=FAKE + 8), "kv_cache is not 16-byte aligned"),
    (dict(kvs=None), "kv_strides"),
    (dict(tks=None), "topk_strides"),
    (dict(tks=(16, 16, -1)), "topk strides"),
    (dict(kvs=(256 * 128, 256 * 128, 256, 2)), "last-dim stride"),
    (dict(kvs=(256 * 128, 256 * 128, 264, 1)), "16 bytes"),
    (dict(kvs=(256 * 128, 256 * 128, 128, 1)), "shorter"),
    (dict(kvs=(0, 256 * 128, 256, 1)), "positive"),
    (dict(nb=0), "num_kv_blocks"),
    (dict(sm=float("nan")), "finite"),
    (dict(ks=float("inf")), "finite"),
    (dict(qs=float("nan")), "finite"),
    (dict(qs=0.0), "positive"),
    (dict(qs=-0.5), "positive"),
    (dict(ks=-1.0), "positive"),
    (dict(sm=0.0), "positive"),
])
def test_run_rejects_bad_arguments(lib, over, fragment):
    h = _plan(lib)
    try:
        st, msg = _run(lib, h, **over)
        assert st == msa.MSA_ERR_INVALID_ARG and fragment in msg, (st, msg)
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


def test_run_null_plan(lib):
    st, msg = _run(lib, None)
    assert st == msa.MSA_ERR_INVALID_ARG and "plan" in msg


def test_bf16_strides_are_checked_in_bytes(lib):
    h = _plan(lib, kv_dtype=msa.KV_BF16)
    try:
        # 260 bf16 elements = 520 bytes: not a multiple of 16 bytes
        st, msg = _run(lib, h, kvs=(260 * 128, 260 * 128, 260, 1))
        assert st == msa.MSA_ERR_INVALID_ARG and "16 bytes" in msg
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


@pytest.mark.parametrize("row_elems,ok", [((1 << 24) - 16, True), (1 << 24, False)])
def test_row_stride_limit_fits_24_bit_offsets(lib, row_elems, ok):
    """The kernels form page-row offsets with 24-bit multiplies, so an fp8 row
    stride of 2^24 bytes (whose low 24 bits are zero) must be rejected, and
    one 16 bytes shorter accepted.  The plan names a device index no machine
    has (a one-split plan makes no HIP call), so an accepted run stops at
    selecting that device, past every argument check, and nothing launches."""
    h = ctypes.c_void_p()
    s = shape()
    assert lib.msa_sparse_decode_plan(ctypes.byref(s), 4096, ctypes.byref(h)) == 0
    try:
        st, msg = _run(lib, h, kvs=(row_elems * 128, row_elems * 128, row_elems, 1))
        if ok:
            assert st == msa.MSA_ERR_DEVICE, (st, msg)
        else:
            assert st == msa.MSA_ERR_UNSUPPORTED and "16 MiB" in msg, (st, msg)
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


MXFP4_SLOT = 128 * (64 + 4)


@pytest.mark.parametrize("kvs,fragment", [
    ((2 * MXFP4_SLOT, 2 * MXFP4_SLOT, MXFP4_SLOT, 2), "last-dim stride"),
    ((2 * MXFP4_SLOT, 2 * MXFP4_SLOT, MXFP4_SLOT + 4, 1), "multiple of 16"),
    ((2 * MXFP4_SLOT, 2 * MXFP4_SLOT, MXFP4_SLOT // 2, 1), "shorter than a slot"),
    ((0, 2 * MXFP4_SLOT, MXFP4_SLOT, 1), "positive"),
    ((2 * MXFP4_SLOT, -16, MXFP4_SLOT, 1), "positive"),
])
def test_mxfp4_strides_are_byte_strides_of_head_slots(lib, kvs, fragment):
    h = _plan(lib, kv_dtype=msa.KV_MXFP4)
    try:
        st, msg = _run(lib, h, kvs=kvs)
        assert st == msa.MSA_ERR_INVALID_ARG and fragment in msg, (st, msg)
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


def test_mxfp4_conversion_rejects_bad_arguments(lib):
    good = msa._I64x4(2 * MXFP4_SLOT, 2 * MXFP4_SLOT, MXFP4_SLOT, 1)
    fn = lib.msa_mxfp4_to_bf16
    assert fn(None, good, 4, 1, FAKE, None) == msa.MSA_ERR_INVALID_ARG
    assert fn(FAKE, good, 4, 1, None, None) == msa.MSA_ERR_INVALID_ARG
    assert fn(FAKE, good, 4, 0, FAKE, None) == msa.MSA_ERR_INVALID_ARG
    assert fn(FAKE, good, 0, 1, FAKE, None) == msa.MSA_ERR_INVALID_ARG
    assert fn(FAKE, good, 4, 1, FAKE + 8, None) == msa.MSA_ERR_INVALID_ARG
    bad = msa._I64x4(2 * MXFP4_SLOT, 2 * MXFP4_SLOT, 100, 1)
    assert fn(FAKE, bad, 4, 1, FAKE, None) == msa.MSA_ERR_INVALID_ARG


def test_binding_mxfp4_cache_view():
    """A (blocks, 2*Hkv, 128, 68) uint8 cache passes byte strides (page, two
    slots per head, K -> V slot, 1) and must be declared as MXFP4."""
    import torch
    kv = torch.empty(3, 8, 128, 68, dtype=torch.uint8)
    assert tuple(msa._kv_strides(kv, msa.KV_MXFP4)) == (8 * MXFP4_SLOT, 2 * MXFP4_SLOT,
                                                         MXFP4_SLOT, 1)
    assert msa._kv_dtype_of(kv, msa.KV_MXFP4) == msa.KV_MXFP4
    with pytest.raises(ValueError, match="does not match"):
        msa._kv_dtype_of(torch.empty(1, dtype=torch.float8_e4m3fn), msa.KV_MXFP4)
    with pytest.raises(ValueError, match="device"):
        msa._check_kv(kv, 4, msa.KV_MXFP4)


def _score(lib, s, **over):
    args = dict(q=FAKE, kv=FAKE, kvs=(256 * 128, 256 * 128, 256, 1), nb=10, qs=1.0, ks=1.0,
                bt=FAKE, sl=FAKE, mb=64, sc=FAKE, scs=(64 * 8, 8, 1), to=FAKE, k=16)
    args.update(over)
    st = lib.msa_block_score_topk(ctypes.byref(s), args["q"], args["kv"],
                                  msa._I64x4(*args["kvs"]), args["nb"], args["qs"], args["ks"],
                                  args["bt"], args["sl"], args["mb"], args["sc"],
                                  msa._I64x3(*args["scs"]), args["to"], args["k"], None)
    return st, lib.msa_last_error().decode()


@pytest.mark.parametrize("over,fragment", [
    (dict(sc=None), "score must be"),
    (dict(mb=0), "max_blocks"),
    (dict(mb=16385), "max_blocks"),
    (dict(k=0), "topk_k"),
    (dict(k=65), "topk_k"),
    (dict(scs=(1, -1, 1)), "score strides"),
    (dict(ks=float("nan")), "finite"),
    (dict(qs=float("inf")), "finite"),
    (dict(qs=0.0), "positive"),
    (dict(q=FAKE + 2), "q must be"),
])
def test_score_topk_rejects_bad_arguments(lib, over, fragment):
    st, msg = _score(lib, shape(batch=2, decode_query_len=4), **over)
    assert st == msa.MSA_ERR_INVALID_ARG and fragment in msg, (st, msg)


def test_score_without_topk_out_checks_everything_else(lib):
    """topk_out = NULL asks for the scores alone (topk_k is then unused); the
    other arguments are still checked before any HIP call."""
    st, msg = _score(lib, shape(batch=2, decode_query_len=4), to=None, k=0, mb=0)
    assert st == msa.MSA_ERR_INVALID_ARG and "max_blocks" in msg
    st, msg = _score(lib, shape(batch=2, decode_query_len=4), to=None, k=0, qs=0.0)
    assert st == msa.MSA_ERR_INVALID_ARG and "positive" in msg


def test_score_topk_validates_shape(lib):
    st, msg = _score(lib, shape(decode_query_len=40))
    assert st == msa.MSA_ERR_INVALID_ARG and "decode_query_len" in msg
    st, msg = _score(lib, shape(kv_dtype=msa.KV_BF16, q_dtype=msa.Q_FP8_E4M3))
    assert st == msa.MSA_ERR_UNSUPPORTED and "fp8 q" in msg
    st, msg = _score(lib, shape(batch=4097))
    assert st == msa.MSA_ERR_UNSUPPORTED and "batch" in msg


def test_topk_select_rejects_bad_arguments(lib):
    scs = msa._I64x3(1, 1, 1)
    assert lib.msa_topk_select(None, scs, 1, 8, 1, FAKE, 4, None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_topk_select(FAKE, scs, 1, 0, 1, FAKE, 4, None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_topk_select(FAKE, scs, 1, 8, 1, FAKE, 0, None) == msa.MSA_ERR_INVALID_ARG
    assert lib.msa_topk_select(FAKE, scs, 0, 8, 1, FAKE, 4, None) == msa.MSA_ERR_INVALID_ARG


def test_fp8_conversion_rejects_bad_arguments(lib):
    for fn in (lib.msa_fp8_e4m3_to_bf16, lib.msa_fp8_e5m2_to_bf16):
        assert fn(None, FAKE, 4, None) == msa.MSA_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, 0, None) == msa.MSA_ERR_INVALID_ARG


def test_destroy_null_is_ok(lib):
    assert lib.msa_sparse_decode_plan_destroy(None) == 0
    assert lib.msa_last_error().decode() == ""


def test_merge_rejects_bad_arguments(lib):
    assert lib.msa_sparse_decode_merge(None, FAKE, 1.0, None) == msa.MSA_ERR_INVALID_ARG
    h = _plan(lib)
    try:
        assert lib.msa_sparse_decode_merge(h, None, 1.0, None) == msa.MSA_ERR_INVALID_ARG
        assert lib.msa_sparse_decode_merge(h, FAKE + 4, 1.0, None) == msa.MSA_ERR_INVALID_ARG
        assert lib.msa_sparse_decode_merge(h, FAKE, float("nan"), None) == \
            msa.MSA_ERR_INVALID_ARG
        # one split: the merge has nothing to do and launches nothing
        assert lib.msa_sparse_decode_merge(h, FAKE, 1.0, None) == 0
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


def test_attend_rejects_bad_arguments(lib):
    h = _plan(lib)
    try:
        kvs = msa._I64x4(256 * 128, 256 * 128, 256, 1)
        tks = msa._I64x3(16, 16, 1)
        st = lib.msa_sparse_decode_attend(h, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, FAKE,
                                          FAKE, tks, None, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG
        st = lib.msa_sparse_decode_attend(h, FAKE, FAKE, kvs, 10, 1.0, -1.0, 1.0, FAKE, FAKE,
                                          FAKE, tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "positive" in lib.msa_last_error().decode()
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


def test_binding_format_checks():
    """The binding maps tensor dtypes to formats and refuses mismatches before
    calling the library (CPU tensors suffice: the checks come first)."""
    import torch
    assert msa._q_dtype_of(torch.empty(1, dtype=torch.bfloat16)) == msa.Q_BF16
    assert msa._q_dtype_of(torch.empty(1, dtype=torch.float8_e4m3fn)) == msa.Q_FP8_E4M3
    with pytest.raises(ValueError):
        msa._q_dtype_of(torch.empty(1, dtype=torch.float16))
    assert msa._kv_dtype_of(torch.empty(1, dtype=torch.float8_e5m2)) == msa.KV_FP8_E5M2
    assert msa._kv_dtype_of(torch.empty(1, dtype=torch.uint8), msa.KV_FP8_E5M2) == \
        msa.KV_FP8_E5M2
    with pytest.raises(ValueError, match="does not match"):
        msa._kv_dtype_of(torch.empty(1, dtype=torch.float8_e4m3fn), msa.KV_FP8_E5M2)


# ---------------------------------------------------------------------------
# prefill plans
# ---------------------------------------------------------------------------

def test_prefill_shape_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct msa_prefill_shape \{(.*?)\} msa_prefill_shape;", text,
                     flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = [n.strip() for grp in re.findall(r"int32_t\s+([\w\s,]+);", body)
             for n in grp.split(",")]
    assert names == [f for f, _ in msa._PrefillShape._fields_]


def prefill_shape(**kw):
    base = dict(num_prefills=3, num_token_rows=505, page_table_stride=9, num_q_heads=64,
                num_kv_heads=4, page_size=128, head_dim=128, topk_blocks=16,
                kv_dtype=msa.KV_FP8_E4M3, q_dtype=msa.Q_BF16, num_splits=1, tile_rows=0)
    base.update(kw)
    return msa._PrefillShape(*[base[f] for f, _ in msa._PrefillShape._fields_])


def prefill_plan_status(lib, s):
    h = ctypes.c_void_p()
    st = lib.msa_sparse_prefill_plan(ctypes.byref(s), 0, ctypes.byref(h))
    msg = lib.msa_last_error().decode()
    if st == 0:
        lib.msa_sparse_decode_plan_destroy(h)
    return st, msg


@pytest.mark.parametrize("field,value,status,fragment", [
    ("num_prefills", 0, msa.MSA_ERR_INVALID_ARG, "num_prefills"),
    ("num_token_rows", 0, msa.MSA_ERR_INVALID_ARG, "num_token_rows"),
    ("page_size", 64, msa.MSA_ERR_UNSUPPORTED, "page_size"),
    ("topk_blocks", 65, msa.MSA_ERR_UNSUPPORTED, "topk_blocks"),
    ("num_kv_heads", 3, msa.MSA_ERR_INVALID_ARG, "multiple"),
    ("kv_dtype", msa.KV_BF16, None, None),
])
def test_prefill_plan_validation(lib, field, value, status, fragment):
    st, msg = prefill_plan_status(lib, prefill_shape(**{field: value}))
    if status is None:
        assert st == 0, msg
    else:
        assert st == status and fragment in msg, (st, msg)


def test_prefill_plan_fp8_q_needs_fp8_cache(lib):
    st, msg = prefill_plan_status(lib, prefill_shape(kv_dtype=msa.KV_BF16,
                                                     q_dtype=msa.Q_FP8_E4M3))
    assert st == msa.MSA_ERR_UNSUPPORTED and "fp8 q" in msg


def test_prefill_and_decode_plans_do_not_mix(lib):
    kvs = msa._I64x4(256 * 128, 256 * 128, 256, 1)
    tks = msa._I64x3(16 * 4, 16, 1)
    hp = ctypes.c_void_p()
    s = prefill_shape()
    assert lib.msa_sparse_prefill_plan(ctypes.byref(s), 0, ctypes.byref(hp)) == 0
    hd = _plan(lib)
    try:
        # a prefill plan refuses the decode entry points, and vice versa
        st = lib.msa_sparse_decode_run(hp, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, FAKE, FAKE,
                                       tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "prefill" in lib.msa_last_error().decode()
        assert lib.msa_sparse_decode_merge(hp, FAKE, 1.0, None) == msa.MSA_ERR_INVALID_ARG
        st = lib.msa_sparse_prefill_run(hd, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, FAKE,
                                        FAKE, FAKE, tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "decode plan" in lib.msa_last_error().decode()
        # NULL chunk boundaries are rejected before any launch
        st = lib.msa_sparse_prefill_run(hp, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, None,
                                        FAKE, FAKE, tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "cu_seqlens_q" in lib.msa_last_error().decode()
        info = msa._Shape()
        assert lib.msa_sparse_decode_plan_info(hp, None, None, ctypes.byref(info)) == 0
        assert info.decode_query_len == 0 and info.batch == 3 and info.num_token_rows == 505
    finally:
        lib.msa_sparse_decode_plan_destroy(hp)
        lib.msa_sparse_decode_plan_destroy(hd)


# ---------------------------------------------------------------------------
# dense decode and multi-row tiles
# ---------------------------------------------------------------------------

def test_dense_plan_rules(lib):
    # dense decode: topk_blocks = 0, on multi-row tiles only
    st, msg = plan_status(lib, shape(topk_blocks=0))
    assert st == 0, msg
    st, msg = plan_status(lib, shape(topk_blocks=0, tile_rows=1))
    assert st == msa.MSA_ERR_UNSUPPORTED and "dense" in msg
    st, msg = prefill_plan_status(lib, prefill_shape(topk_blocks=0))
    assert st == msa.MSA_ERR_UNSUPPORTED and "prefill" in msg


def test_plan_tile_choice_is_reported():
    """The plan's kernel choice (the measured faster one): single rows for short
    sparse decode, 2-row tiles for long decode query lengths and prefill, 4-row
    tiles for dense decode."""
    cases = [(dict(dql=4, topk=16), 1), (dict(dql=32, topk=16), 2), (dict(dql=4, topk=0), 4),
             (dict(dql=1, topk=0), 2), (dict(dql=8, topk=0), 4)]
    for kw, rows in cases:
        plan = msa.msa_sparse_decode_plan(16, kw["dql"], num_q_heads=64, num_kv_heads=4,
                                          page_table_stride=64, topk_blocks=kw["topk"],
                                          kv_dtype=msa.KV_FP8_E4M3, num_splits=1, device=0)
        assert plan.tile_rows == rows and plan.dense == (kw["topk"] == 0), kw
        plan.close()
    plan = msa.msa_sparse_prefill_plan(3, 505, num_q_heads=16, num_kv_heads=1,
                                       page_table_stride=9, topk_blocks=16,
                                       kv_dtype=msa.KV_FP8_E4M3, num_splits=1, device=0)
    assert plan.tile_rows == 2 and plan.prefill
    plan.close()


def test_dense_and_sparse_runs_check_topk(lib):
    kvs = msa._I64x4(256 * 128, 256 * 128, 256, 1)
    tks = msa._I64x3(16, 16, 1)
    hd = _plan(lib, topk_blocks=0)
    hs = _plan(lib)
    try:
        st = lib.msa_sparse_decode_run(hd, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, FAKE, FAKE,
                                       tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "topk = NULL" in lib.msa_last_error().decode()
        st = lib.msa_sparse_decode_run(hs, FAKE, FAKE, kvs, 10, 1.0, 1.0, 1.0, FAKE, FAKE, None,
                                       tks, FAKE, 0.08, None)
        assert st == msa.MSA_ERR_INVALID_ARG and "topk" in lib.msa_last_error().decode()
    finally:
        lib.msa_sparse_decode_plan_destroy(hd)
        lib.msa_sparse_decode_plan_destroy(hs)


def test_xcd_deal_visits_every_unit_once(tmp_path):
    """The single-row attend and the merge kernel map workgroups to units
    through msa_internal.h's chunked XCD deal: compiled for the host, it must
    visit every unit exactly once (a unit it skipped would never be written)."""
    import shutil
    import subprocess

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "xcd_cover"
    subprocess.run([hipcc, "-std=c++17", "-O1",
                    "-I", os.path.join(root, "block_sparse_gqa_decode_amd", "csrc"),
                    os.path.join(root, "tests", "host", "xcd_cover.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=300)
    assert out.stdout.strip() == "ok"


def test_c_consumer_links_and_reports_misuse():
    """The plain C consumer of the ABI (tests/host/c_abi_decode.c, built by
    build()) links against the library, checks msa_abi_version and sees a
    decode_query_len of 33 rejected with a message, all before touching a
    device.  Without a GPU it then stops at its first hipMalloc (exit 2); on a
    GPU machine the GPU test runs it to the end."""
    import subprocess

    from block_sparse_gqa_decode_amd import build_lib

    exe = build_lib.C_CONSUMER_BIN
    if not os.path.exists(exe):
        build_lib.build_c_consumer()
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 2, (res.returncode, res.stdout, res.stderr)
    assert "hipMalloc" in res.stderr and "not rejected" not in res.stderr, res.stderr


def test_read_runs_probe_rejects_bad_arguments(lib):
    f = lib.msa_probe_read_runs
    ok = dict(base=FAKE, nbytes=1 << 20, off=FAKE, ln=FAKE, nruns=4, first=FAKE, wgs=2,
              out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["base"], a["nbytes"], a["off"], a["ln"], a["nruns"], a["first"], a["wgs"],
                 a["out"], None)

    assert call(wgs=-1) == msa.MSA_ERR_INVALID_ARG
    assert call(nruns=-1) == msa.MSA_ERR_INVALID_ARG
    assert call(base=None) == msa.MSA_ERR_INVALID_ARG
    assert call(out=None) == msa.MSA_ERR_INVALID_ARG
    assert call(first=None) == msa.MSA_ERR_INVALID_ARG
    assert call(off=None) == msa.MSA_ERR_INVALID_ARG
    assert call(base=FAKE + 8) == msa.MSA_ERR_INVALID_ARG
    assert "aligned" in lib.msa_last_error().decode()
    assert call(nbytes=8) == msa.MSA_ERR_INVALID_ARG
    assert call(wgs=1 << 25) == msa.MSA_ERR_UNSUPPORTED
    # No workgroups: nothing to launch, so no HIP call and no error.
    assert call(wgs=0, base=None) == msa.MSA_OK


def test_noalloc_rejects_partials_beyond_its_scratch(lib):
    """The no-allocation entry point checks the static scratch size on the
    host, before any HIP call: 4096 rows x 64 q heads x 16 splits of partials
    (about 2.2 GB) exceed its 64 MiB."""
    s = shape(batch=128, decode_query_len=32, num_q_heads=64, num_kv_heads=4, num_splits=16)
    strides = (ctypes.c_int64 * 4)(4 * 128 * 256, 128 * 256, 256, 1)
    tk = (ctypes.c_int64 * 3)(64, 16, 1)
    st = lib.msa_sparse_decode_run_noalloc(ctypes.byref(s), 0, None, None, strides, 1, 1.0,
                                           1.0, 1.0, None, None, None, tk, None, 0.1, None)
    assert st == -2
    msg = lib.msa_last_error().decode()
    assert "static scratch" in msg and "67108864" in msg
    bad = shape(decode_query_len=33)
    st = lib.msa_sparse_decode_run_noalloc(ctypes.byref(bad), 0, None, None, strides, 1, 1.0,
                                           1.0, 1.0, None, None, None, tk, None, 0.1, None)
    assert st == -1 and "decode_query_len" in lib.msa_last_error().decode()


def test_eight_row_tiles_need_an_8bit_cache(lib):
    """8-row tiles stage fp8 pages through LDS: a bf16 or MXFP4 cache is refused
    before any HIP call; e4m3 and e5m2 are accepted."""
    for kvd in (msa.KV_BF16, msa.KV_MXFP4):
        st, msg = plan_status(lib, shape(tile_rows=8, kv_dtype=kvd))
        assert st == msa.MSA_ERR_UNSUPPORTED and "8-row tiles" in msg, (kvd, st, msg)
    for kvd in (msa.KV_FP8_E4M3, msa.KV_FP8_E5M2):
        st, msg = plan_status(lib, shape(tile_rows=8, kv_dtype=kvd, num_splits=1))
        assert st == 0, (kvd, msg)


def _select_run(lib, h, **over):
    args = dict(q=FAKE, kv=FAKE, kvs=(256 * 128, 256 * 128, 256, 1), nb=10, bt=FAKE, sl=FAKE,
                sc=FAKE, scs=(64 * 16, 16, 1), mb=64, tko=None, out=FAKE, sm=0.088)
    args.update(over)
    kvs = msa._I64x4(*args["kvs"])
    scs = msa._I64x3(*args["scs"]) if args["scs"] is not None else None
    st = lib.msa_sparse_decode_select_run(h, args["q"], args["kv"], kvs, args["nb"], 1.0, 1.0,
                                          1.0, args["bt"], args["sl"], args["sc"], scs,
                                          args["mb"], args["tko"], args["out"], args["sm"],
                                          None)
    return st, lib.msa_last_error().decode()


@pytest.mark.parametrize("over,fragment", [
    (dict(sc=None), "score"),
    (dict(scs=None), "score_strides"),
    (dict(scs=(64 * 16, -16, 1)), "score strides"),
    (dict(mb=0), "max_blocks"),
    (dict(mb=16385), "max_blocks"),
    (dict(q=None), "q and out"),
    (dict(bt=None), "block_table"),
])
def test_select_run_rejects_bad_arguments(lib, over, fragment):
    h = _plan(lib)
    try:
        st, msg = _select_run(lib, h, **over)
        assert st == msa.MSA_ERR_INVALID_ARG and fragment in msg, (st, msg)
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


@pytest.mark.parametrize("kw", [dict(topk_blocks=0), dict(decode_query_len=8, tile_rows=2)])
def test_select_run_needs_a_single_row_sparse_plan(lib, kw):
    """The selecting attend is the single-row kernel's; a dense plan or a
    row-tile plan is refused before any HIP call."""
    h = _plan(lib, **kw)
    try:
        st, msg = _select_run(lib, h)
        assert st == msa.MSA_ERR_UNSUPPORTED and "single-row" in msg, (st, msg)
    finally:
        lib.msa_sparse_decode_plan_destroy(h)


def test_select_run_refuses_a_prefill_plan(lib):
    plan = msa.msa_sparse_prefill_plan(2, 40, num_q_heads=16, num_kv_heads=1,
                                       page_table_stride=10, topk_blocks=8,
                                       kv_dtype=msa.KV_FP8_E4M3, num_splits=1, device=0)
    try:
        st, msg = _select_run(lib, plan.handle)
        assert st == msa.MSA_ERR_INVALID_ARG and "prefill" in msg
    finally:
        plan.close()
