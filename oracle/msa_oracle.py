"""Float64 CPU oracle for block-sparse GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product path
(the HIP library and its binding) never routes through it, and it shares no
code, table or helper with that path.

What it computes, written out from the pages' definitions with no blocking,
fusion or reordering:

* ``sparse_decode`` -- each decode query token attends, per kv head, only the
  keys of its selected 128-token pages that are causally visible at its
  position (vLLM API page ``vllm.models.minimax_m3.common.sparse_attention``:
  ``MiniMaxM3SparseImpl`` docstring and ``MiniMaxM3SparseTritonImpl.forward``;
  vLLM test file ``test_minimax_m3_msa_cutlass_sparse_decode.py``:
  ``_make_topk``).  Steps: dequant -> gather the selected live pages -> causal
  mask -> softmax -> PV.
* ``block_max_scores`` -- the indexer's per-block causal max of q.k over the
  group's q heads and visible keys (TensorRT-LLM PR #17171 "Custom decode
  kernels for MinimaxM3", indexer-scorer commit message).
* ``select_topk`` -- top-k blocks per (token, kv head) by score, ties to the
  lower block index, padded with -1 (same PR, selector; tie rule from the
  full-decode-step workload statement).
* ``dense_decode`` -- the decode attend over every causally visible block
  (TensorRT-LLM PR #17171, dense-decode commit: M3's first layers attend the
  whole page table).
* ``sparse_prefill`` -- the same attend for ragged prefill chunks: request r
  owns token rows ``cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1`` and its local
  token i sits at ``context_lens[r] + i`` (vLLM sparse-attention page,
  ``MiniMaxM3SparsePrefillMetadata`` and the prefill call of
  ``MiniMaxM3SparseTritonImpl.forward``; the test page's prefill test builds
  ``context_lens = seq_lens - q_lens`` and selects every visible page up to
  ``(seq_len - q_len + local_q) // 128``).

Readings taken where the pages leave a step open (each is also listed in the
design notes):

1. Top-k entries are *logical* block ids into the request's block-table row
   (``_make_topk`` writes ``arange(visible_pages)`` over a shuffled pool).
2. Token ``t = r*dql + l`` sits at ``pos = seq_len[r] - dql + l`` and sees keys
   ``0..pos`` (``_make_topk``: ``visible_tokens = seq_len - query_len +
   local_query + 1``).
3. A negative index, or a block that starts after ``pos``, contributes nothing
   and its block-table entry is not read.  So does a block id at or beyond
   the block-table row, or a block whose table entry is not a page of the
   pool (outside ``[0, num_blocks)``); the scorer leaves such a block at
   ``-inf``.  The pages do not say what a bad table entry means; this is the
   library boundary's rule for data-dependent inputs, which never index out
   of the pool.
4. A row with no visible key (all -1, or a padding row ``t >= batch*dql``)
   outputs exact zeros (PR #17171, flash-decoding commit: zeroed, not NaN,
   output for padding rows).
5. q head ``j`` reads kv head ``j // G`` with ``G = Hq / Hkv``.
6. KV bytes are OCP fp8 e4m3fn (``torch.float8_e4m3fn`` in the test file),
   OCP fp8 e5m2 (the backend's ``supported_kv_cache_dtypes`` lists
   ``fp8_e5m2``; ``MiniMaxM3SparseTritonImpl`` picks ``torch.float8_e5m2`` off
   fnuz platforms, and gfx950 uses the OCP formats) or bf16; K is the first 128
   entries of the packed last dim, V the last 128 (``msa_cutlass_sparse_decode``:
   ``kv_cache.split(_HEAD_DIM, dim=-1)``).  ``k_scale``/``v_scale`` multiply the
   decoded values.
7. The scorer uses the attention q and the K half of the same cache, raw dot
   product (no softmax scale), ``-inf`` for blocks that start after ``pos``.
8. The selector ranks blocks with score ``> -inf`` by (score desc, block asc).
9. q is bf16, or OCP fp8 e4m3fn codes with a per-tensor ``q_scale``: the value
   is ``decode(code) * q_scale`` (``msa_cutlass_sparse_decode(query_fp8, ...,
   q_scale_float, ...)``; the test file compares it with the bf16 path fed
   ``query_fp8.to(bfloat16) * q_scale``).  A bf16 q is multiplied by
   ``q_scale`` too (1 by default).
10. Prefill token rows at or past ``cu_seqlens_q[-1]`` are padding rows
    (zeros); a request with ``q_len = 0`` owns no row.
11. The 4-bit cache is an MXFP4 analogue of the pages' NVFP4 cache (vLLM
    test file, ``_make_nvfp4_kv_cache`` and
    ``test_nvfp4_kv_cache_views_address_head_slots``).  Kept from the pages:
    a page holds ``2*Hkv`` head slots; slot ``2h`` is K of kv head h and slot
    ``2h+1`` its V, so a head is one contiguous run of the page; a slot holds
    the 128 rows' packed 4-bit data, then the 128 rows' block scales; a
    per-tensor global ``k_scale`` / ``v_scale`` applies on top.  Changed for
    the OCP MX formats gfx950 decodes natively: elements are OCP e2m1
    (``±{0, 0.5, 1, 1.5, 2, 3, 4, 6}``), one E8M0 scale ``2^(E-127)``
    (``E = 255`` is NaN) covers 32 consecutive head dims of a row (4 bytes
    per row instead of NVFP4's 8 e4m3 scales per 16), V scales are stored
    row-linear like K's (NVFP4's swizzle is a tensor-core layout), element
    ``2i`` of a row sits in the low nibble of byte ``i``, and the global
    scales multiply, as ``k_scale`` / ``v_scale`` do for fp8.  A value is
    ``e2m1 * 2^(E-127) * k_scale`` (resp. ``v_scale``).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
something other than itself (torch's fp8/bf16/E8M0 casts, the OCP MX FP4
value table, dense causal attention
through ``torch.nn.functional.scaled_dot_product_attention``, closed forms,
invariances, brute-force loops).
"""
from __future__ import annotations

import math

import numpy as np

PAGE = 128
HEAD_DIM = 128


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def decode_e4m3fn(codes) -> np.ndarray:
    """OCP fp8 e4m3fn code -> float64 value.

    Bit fields: sign s (bit 7), exponent E (bits 6..3, bias 7), mantissa M
    (bits 2..0).  E == 15 and M == 7 is NaN (no infinities); E == 0 is
    subnormal ``M/8 * 2^-6``; otherwise ``(1 + M/8) * 2^(E-7)``.  Largest
    finite magnitude 448.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    nor = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = np.where(e == 0, sub, nor)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return v.astype(np.float64)


_E4M3_TABLE = decode_e4m3fn(np.arange(256))


def decode_e5m2(codes) -> np.ndarray:
    """OCP fp8 e5m2 code -> float64 value.

    Bit fields: sign s (bit 7), exponent E (bits 6..2, bias 15), mantissa M
    (bits 1..0).  E == 31 is +-inf when M == 0 and NaN otherwise; E == 0 is
    subnormal ``M/4 * 2^-14``; otherwise ``(1 + M/4) * 2^(E-15)``.  Largest
    finite magnitude 57344.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 2) & 0x1F
    m = c & 0x3
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 4.0) * 2.0 ** -14
    nor = sign * (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15.0)
    v = np.where(e == 0, sub, nor)
    v = np.where((e == 31) & (m == 0), sign * np.inf, v)
    v = np.where((e == 31) & (m != 0), np.nan, v)
    return v.astype(np.float64)


_E5M2_TABLE = decode_e5m2(np.arange(256))


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float64 (exact: bf16 is the top half of an
    fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e2m1(codes) -> np.ndarray:
    """OCP FP4 e2m1 code (low 4 bits) -> float64 value.

    Bit fields: sign s (bit 3), exponent E (bits 2..1, bias 1), mantissa M
    (bit 0).  E == 0 is subnormal ``M/2``; otherwise ``(1 + M/2) * 2^(E-1)``.
    No infinities or NaN; largest magnitude 6.
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 2.0)
    nor = sign * (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    return np.where(e == 0, sub, nor).astype(np.float64)


def decode_e8m0(codes) -> np.ndarray:
    """OCP E8M0 scale code -> float64 ``2^(E-127)``; code 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    v = np.exp2(c.astype(np.float64) - 127.0)
    return np.where(c == 255, np.nan, v)


MXFP4_BLOCK = 32                                   # head dims per E8M0 scale
MXFP4_DATA_BYTES = PAGE * HEAD_DIM // 2            # 128 rows x 64 bytes
MXFP4_SLOT_BYTES = MXFP4_DATA_BYTES + PAGE * HEAD_DIM // MXFP4_BLOCK   # + 128 x 4


def mxfp4_slot(kv: np.ndarray, page: int, head: int, side: int):
    """The (data [128, 64], scales [128, 4]) bytes of one head slot of a 4-bit
    page (reading 11): slot ``2*head + side``, side 0 = K, 1 = V."""
    flat = np.asarray(kv[int(page), 2 * int(head) + int(side)]).reshape(-1)
    assert flat.size == MXFP4_SLOT_BYTES
    data = flat[:MXFP4_DATA_BYTES].reshape(PAGE, HEAD_DIM // 2)
    scales = flat[MXFP4_DATA_BYTES:].reshape(PAGE, HEAD_DIM // MXFP4_BLOCK)
    return data, scales


def mxfp4_rows(data: np.ndarray, scales: np.ndarray, n: int) -> np.ndarray:
    """The first n rows of a 4-bit slot as float64 [n, 128]: element d of a
    row is nibble ``d % 2`` (low first) of byte ``d // 2``, times the scale
    of block ``d // 32``."""
    d = np.arange(HEAD_DIM)
    byte = data[:n, d // 2].astype(np.int64)
    code = (byte >> (4 * (d % 2))) & 0xF
    return decode_e2m1(code) * decode_e8m0(scales[:n, d // MXFP4_BLOCK])


def page_kv(kv, kv_dtype: str, k_scale: float, v_scale: float, page: int, head: int,
            n: int):
    """Dequantized K and V rows 0..n-1 of one (page, kv head), float64."""
    if kv_dtype == "mxfp4":
        kd, ks = mxfp4_slot(kv, page, head, 0)
        vd, vs = mxfp4_slot(kv, page, head, 1)
        return (mxfp4_rows(kd, ks, n) * float(k_scale),
                mxfp4_rows(vd, vs, n) * float(v_scale))
    kraw, vraw = split_kv(kv[page, head, :n, :])
    return dequant(kraw, kv_dtype, k_scale), dequant(vraw, kv_dtype, v_scale)


def dequant(raw: np.ndarray, kv_dtype: str, scale: float) -> np.ndarray:
    """Stored KV entries -> float64 values times the per-tensor scale."""
    if kv_dtype == "fp8_e4m3":
        return _E4M3_TABLE[np.asarray(raw, dtype=np.uint8)] * float(scale)
    if kv_dtype == "fp8_e5m2":
        return _E5M2_TABLE[np.asarray(raw, dtype=np.uint8)] * float(scale)
    if kv_dtype == "bf16":
        return decode_bf16(raw) * float(scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def decode_query(q, q_dtype: str, q_scale: float) -> np.ndarray:
    """Stored q entries (bf16 bits, or fp8 e4m3fn codes) -> float64 values
    times the per-tensor q scale (reading 9)."""
    if q_dtype == "bf16":
        return decode_bf16(q) * float(q_scale)
    if q_dtype == "fp8_e4m3":
        return _E4M3_TABLE[np.asarray(q, dtype=np.uint8)] * float(q_scale)
    raise ValueError(f"unknown q dtype {q_dtype!r}")


# ---------------------------------------------------------------------------
# indexing helpers (small on purpose: the pin tests plant mistakes in them)
# ---------------------------------------------------------------------------

def token_position(seq_len: int, dql: int, local: int) -> int:
    """Absolute 0-based position of local decode token ``local``."""
    return int(seq_len) - int(dql) + int(local)


def visible_rows(pos: int, block: int) -> int:
    """Number of keys of logical block ``block`` visible at ``pos``
    (0 when the block starts after ``pos``)."""
    if block < 0 or block * PAGE > pos:
        return 0
    return min(PAGE, pos - block * PAGE + 1)


def kv_head_of(q_head: int, group: int) -> int:
    return q_head // group


def split_kv(raw_rows: np.ndarray):
    """Packed rows [n, 2*D] -> (K rows, V rows)."""
    return raw_rows[:, :HEAD_DIM], raw_rows[:, HEAD_DIM:]


def softmax_attend(qv: np.ndarray, k: np.ndarray, v: np.ndarray,
                   sm_scale: float) -> np.ndarray:
    """softmax(sm_scale * q k^T) v for one query vector, float64."""
    z = sm_scale * (k @ qv)
    z = z - z.max()
    w = np.exp(z)
    return (w @ v) / w.sum()


# ---------------------------------------------------------------------------
# the attend
# ---------------------------------------------------------------------------

def gather_live(kv, kv_dtype, k_scale, v_scale, block_table_row, pos, head,
                indices, check_distinct=True):
    """Dequantized K and V rows of the selected blocks visible at ``pos``."""
    ks, vs, seen = [], [], set()
    for b in indices:
        b = int(b)
        n = visible_rows(pos, b)
        if n <= 0:
            continue
        if check_distinct:
            assert b not in seen, f"duplicate block index {b}"
            seen.add(b)
        if b >= len(block_table_row):
            continue
        p = int(block_table_row[b])
        if p < 0 or p >= kv.shape[0]:
            continue
        k, v = page_kv(kv, kv_dtype, k_scale, v_scale, p, head, n)
        ks.append(k)
        vs.append(v)
    if not ks:
        return None, None
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def sparse_decode(q_bits, kv, kv_dtype, k_scale, v_scale, block_table, seq_lens,
                  topk, decode_query_len, num_kv_heads, sm_scale, rows=None,
                  q_dtype="bf16", q_scale=1.0):
    """Block-sparse GQA decode, float64.

    q_bits   uint16 bf16 bits, or uint8 fp8 e4m3fn codes (``q_dtype``),
             [num_token_rows, Hq, 128]; values times ``q_scale``
    kv       uint8 (fp8 codes) or uint16 (bf16 bits) [num_blocks, Hkv, 128, 256],
             or uint8 [num_blocks, 2*Hkv, 128, 68] 4-bit head slots (reading 11)
    topk     int32 [num_token_rows, Hkv, k] logical block ids (-1 = none)
    rows     optional iterable of token rows to evaluate (default: all)

    Returns float64 [len(rows), Hq, 128].  Rows at or past
    ``batch*decode_query_len`` are padding rows and come back as zeros.
    """
    q_bits = np.asarray(q_bits)
    num_rows, hq, d = q_bits.shape
    assert d == HEAD_DIM and hq % num_kv_heads == 0
    group = hq // num_kv_heads
    dql = int(decode_query_len)
    real = len(seq_lens) * dql
    row_list = range(num_rows) if rows is None else list(rows)
    out = np.zeros((len(row_list), hq, HEAD_DIM), dtype=np.float64)
    for i, t in enumerate(row_list):
        if t >= real:
            continue
        r, loc = divmod(int(t), dql)
        pos = token_position(seq_lens[r], dql, loc)
        gathered = {}
        for j in range(hq):
            h = kv_head_of(j, group)
            if h not in gathered:
                gathered[h] = gather_live(kv, kv_dtype, k_scale, v_scale,
                                          block_table[r], pos, h, topk[t, h, :])
            k, v = gathered[h]
            if k is None:
                continue
            qv = decode_query(q_bits[t, j], q_dtype, q_scale)
            out[i, j] = softmax_attend(qv, k, v, sm_scale)
    return out


def dense_decode(q_bits, kv, kv_dtype, k_scale, v_scale, block_table, seq_lens,
                 decode_query_len, num_kv_heads, sm_scale, rows=None, q_dtype="bf16",
                 q_scale=1.0):
    """Decode attend over all keys 0..pos of the request's pages (no top-k),
    float64.  Padding rows, and rows with no live key (a position before the
    first key, or every visible block outside the pool), are zeros, as in
    ``sparse_decode``.  Returns float64 [len(rows), Hq, 128]."""
    q_bits = np.asarray(q_bits)
    num_rows, hq, d = q_bits.shape
    assert d == HEAD_DIM and hq % num_kv_heads == 0
    group = hq // num_kv_heads
    dql = int(decode_query_len)
    real = len(seq_lens) * dql
    row_list = range(num_rows) if rows is None else list(rows)
    out = np.zeros((len(row_list), hq, HEAD_DIM), dtype=np.float64)
    for i, t in enumerate(row_list):
        if t >= real:
            continue
        r, loc = divmod(int(t), dql)
        pos = token_position(seq_lens[r], dql, loc)
        every = range(pos // PAGE + 1)
        gathered = {}
        for j in range(hq):
            h = kv_head_of(j, group)
            if h not in gathered:
                gathered[h] = gather_live(kv, kv_dtype, k_scale, v_scale,
                                          block_table[r], pos, h, every)
            k, v = gathered[h]
            if k is None:      # no live key (pos < 0, or no block in the pool)
                continue
            qv = decode_query(q_bits[t, j], q_dtype, q_scale)
            out[i, j] = softmax_attend(qv, k, v, sm_scale)
    return out


def prefill_request_of(cu_seqlens_q, t: int):
    """The request whose row range [cu[r], cu[r+1]) holds token row t, or
    None for a padding row."""
    cu = [int(x) for x in cu_seqlens_q]
    for r in range(len(cu) - 1):
        if cu[r] <= t < cu[r + 1]:
            return r
    return None


def prefill_position(context_len: int, row_start: int, t: int) -> int:
    """Absolute position of prefill token row t of a request whose rows start
    at ``row_start`` after ``context_len`` cached tokens."""
    return int(context_len) + int(t) - int(row_start)


def sparse_prefill(q_bits, kv, kv_dtype, k_scale, v_scale, block_table, cu_seqlens_q,
                   context_lens, topk, num_kv_heads, sm_scale, rows=None,
                   q_dtype="bf16", q_scale=1.0):
    """Block-sparse GQA attend over ragged prefill chunks, float64.

    Token row t of request r (``cu_seqlens_q[r] <= t < cu_seqlens_q[r+1]``)
    sits at ``pos = context_lens[r] + t - cu_seqlens_q[r]`` and attends the
    keys 0..pos of its selected blocks; everything else is as in
    ``sparse_decode``.  Returns float64 [len(rows), Hq, 128].
    """
    q_bits = np.asarray(q_bits)
    num_rows, hq, d = q_bits.shape
    assert d == HEAD_DIM and hq % num_kv_heads == 0
    group = hq // num_kv_heads
    row_list = range(num_rows) if rows is None else list(rows)
    out = np.zeros((len(row_list), hq, HEAD_DIM), dtype=np.float64)
    for i, t in enumerate(row_list):
        r = prefill_request_of(cu_seqlens_q, int(t))
        if r is None:
            continue
        pos = prefill_position(context_lens[r], cu_seqlens_q[r], t)
        gathered = {}
        for j in range(hq):
            h = kv_head_of(j, group)
            if h not in gathered:
                gathered[h] = gather_live(kv, kv_dtype, k_scale, v_scale,
                                          block_table[r], pos, h, topk[t, h, :])
            k, v = gathered[h]
            if k is None:
                continue
            qv = decode_query(q_bits[t, j], q_dtype, q_scale)
            out[i, j] = softmax_attend(qv, k, v, sm_scale)
    return out


# ---------------------------------------------------------------------------
# the indexer block-max scorer and the top-k selector
# ---------------------------------------------------------------------------

def block_max_scores(q_bits, kv, kv_dtype, k_scale, block_table, seq_lens,
                     decode_query_len, num_kv_heads, max_blocks, rows=None,
                     q_dtype="bf16", q_scale=1.0):
    """score[h, b, t] = max over the group's q heads g and the visible keys j
    of block b of q[t, h*G+g] . K[page(b), h, j]; -inf where block b starts
    after token t's position.  Raw dot product (no softmax scale).

    Returns float64 [Hkv, max_blocks, len(rows)].
    """
    q_bits = np.asarray(q_bits)
    num_rows, hq, _ = q_bits.shape
    group = hq // num_kv_heads
    dql = int(decode_query_len)
    real = len(seq_lens) * dql
    row_list = range(min(num_rows, real)) if rows is None else list(rows)
    score = np.full((num_kv_heads, max_blocks, len(row_list)), -np.inf)
    for i, t in enumerate(row_list):
        if t >= real:
            continue
        r, loc = divmod(int(t), dql)
        pos = token_position(seq_lens[r], dql, loc)
        for h in range(num_kv_heads):
            qs = decode_query(q_bits[t, h * group:(h + 1) * group], q_dtype,
                              q_scale)                               # [G, D]
            for b in range(max_blocks):
                n = visible_rows(pos, b)
                if n <= 0:
                    continue
                p = int(block_table[r, b]) if b < block_table.shape[1] else -1
                if p < 0 or p >= kv.shape[0]:
                    continue                                     # stays -inf
                k, _ = page_kv(kv, kv_dtype, k_scale, 1.0, p, h, n)  # [n, D]
                score[h, b, i] = np.max(qs @ k.T)
    return score


def select_topk(score, k: int) -> np.ndarray:
    """score [Hkv, NB, T] -> int32 [T, Hkv, k]: blocks with score > -inf ranked
    by (score descending, block id ascending), first k, padded with -1."""
    score = np.asarray(score, dtype=np.float64)
    hkv, nb, nt = score.shape
    out = np.full((nt, hkv, k), -1, dtype=np.int32)
    for h in range(hkv):
        for t in range(nt):
            s = score[h, :, t]
            cand = [b for b in range(nb) if s[b] > -math.inf]
            cand.sort(key=lambda b: (-s[b], b))
            sel = cand[:k]
            out[t, h, :len(sel)] = sel
    return out
