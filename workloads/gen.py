"""Seeded synthetic inputs for block-sparse GQA decode.

This module is shared by the float64 oracle tests and by the HIP path tests and
bench.  It holds none of the method's arithmetic: only random draws (NumPy
PCG64), page-table construction, index-list construction and the encoding of
drawn values into bf16 / OCP fp8 e4m3fn bit patterns (done by torch's CPU
casts, round-to-nearest-even).

Shapes and structure follow the workloads the pages describe:

* KV cache: vLLM API page ``vllm.models.minimax_m3.common.sparse_attention``,
  ``MiniMaxM3SparseBackend.get_kv_cache_shape`` -- logical
  ``(num_blocks, num_kv_heads, block_size=128, 2*head_size)`` with K in the
  first 128 entries of the last dim and V in the last 128, HND stride order.
* Paged layout over a shuffled physical pool and the "every visible page"
  index pattern: vLLM test file
  ``test_minimax_m3_msa_cutlass_sparse_decode.py``, helpers
  ``_make_paged_layout`` and ``_make_topk``.
* Token row ``t = request * dql + local`` at position
  ``seq_len - dql + local`` (same test file, ``_make_topk``).
* An fp8 query: e4m3fn codes of ``q / q_scale`` with a per-tensor scale (the
  test file quantizes the bf16 query with ``scaled_fp8_quant`` and a given
  scale before ``msa_cutlass_sparse_decode``).

* A 4-bit cache: the pages' NVFP4 head-slot page (test file,
  ``_make_nvfp4_kv_cache``: slot 2h = K of head h, slot 2h+1 = V, each the
  rows' packed data then their block scales), with OCP MXFP4 elements (e2m1,
  one E8M0 scale per 32 head dims, element 2i in the low nibble of byte i).
  The block scale of 32 values is the OCP MX choice
  ``2^(floor(log2(amax)) - 2)``; elements round to the nearest e2m1 value
  (ties to the smaller magnitude), saturating at 6.

Every array is plain NumPy: fp8 codes as ``uint8``, bf16 as ``uint16`` bit
patterns, indices as ``int32``.  fp8 e5m2 KV codes are ``uint8`` too; a 4-bit
pool is ``uint8 [num_blocks, 2*Hkv, 128, 68]`` (each slot's 8704 bytes).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE = 128
HEAD_DIM = 128
FP8_MAX = 448.0
E5M2_MAX = 57344.0
BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F      # NaN in both e4m3fn (E=15, M=7) and e5m2 (E=31, M=3)

KV_FP8 = "fp8_e4m3"
KV_E5M2 = "fp8_e5m2"
KV_BF16 = "bf16"
KV_8BIT = (KV_FP8, KV_E5M2)
KV_MXFP4 = "mxfp4"
MXFP4_BLOCK = 32
MXFP4_DATA_BYTES = PAGE * HEAD_DIM // 2
MXFP4_SLOT_BYTES = MXFP4_DATA_BYTES + PAGE * HEAD_DIM // MXFP4_BLOCK
MXFP4_NAN_SCALE = 0xFF
_E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
Q_BF16 = "bf16"
Q_FP8 = "fp8_e4m3"


# ---------------------------------------------------------------------------
# encoders (torch CPU casts; no attention arithmetic)
# ---------------------------------------------------------------------------

def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float array -> bf16 bit patterns (uint16), round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float array -> OCP fp8 e4m3fn codes (uint8), clipped to +-448 first."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp(-FP8_MAX, FP8_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def encode_e5m2(x: np.ndarray) -> np.ndarray:
    """float array -> OCP fp8 e5m2 codes (uint8), clipped to +-57344 first."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp(-E5M2_MAX, E5M2_MAX)
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy().copy()


def encode_mxfp4(x: np.ndarray):
    """float rows [..., 128] -> (packed e2m1 data uint8 [..., 64], E8M0 block
    scales uint8 [..., 4]).  Input generation only: any valid encoding is a
    valid input, and the oracle decodes whatever bytes this writes."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    blk = x.reshape(lead + (HEAD_DIM // MXFP4_BLOCK, MXFP4_BLOCK))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = f * 2^ex, f in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1 - 2 + 127, 1, 254)
    e = np.where(amax > 0, e, 127)
    y = blk / np.exp2(e - 127).astype(np.float32)[..., None]
    mag = np.searchsorted(_E2M1_MIDPOINTS, np.abs(y), side="left").astype(np.uint8)
    code = mag | np.where((y < 0) & (mag > 0), 8, 0).astype(np.uint8)
    code = code.reshape(lead + (HEAD_DIM,))
    data = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return data, e.astype(np.uint8)


def pack_mxfp4_pages(x: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Packed K|V values ``[pages, Hkv, 128, 256]`` -> 4-bit head-slot pages
    ``uint8 [pages, 2*Hkv, 128, 68]``: slot 2h holds head h's K rows, slot
    2h+1 its V rows, each as 128 x 64 data bytes then 128 x 4 scale bytes."""
    pages, hkv = x.shape[0], x.shape[1]
    if out is None:
        out = np.empty((pages, 2 * hkv, PAGE, MXFP4_SLOT_BYTES // PAGE), dtype=np.uint8)
    slots = out.reshape(pages, hkv, 2, MXFP4_SLOT_BYTES)
    for side in range(2):
        data, scales = encode_mxfp4(x[..., side * HEAD_DIM:(side + 1) * HEAD_DIM])
        slots[:, :, side, :MXFP4_DATA_BYTES] = data.reshape(pages, hkv, -1)
        slots[:, :, side, MXFP4_DATA_BYTES:] = scales.reshape(pages, hkv, -1)
    return out


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _encode(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == KV_FP8:
        return encode_e4m3fn(x)
    if kv_dtype == KV_E5M2:
        return encode_e5m2(x)
    return encode_bf16(x)


# ---------------------------------------------------------------------------
# case container
# ---------------------------------------------------------------------------

@dataclass
class DecodeCase:
    """One decode step's inputs (optionally with extra (q, topk) replicas)."""

    name: str
    seed: int
    batch: int
    dql: int
    num_token_rows: int
    num_q_heads: int
    num_kv_heads: int
    topk_k: int
    kv_dtype: str
    seq_lens: np.ndarray           # int32 [batch]
    block_table: np.ndarray        # int32 [batch, stride]
    kv: np.ndarray                 # uint8 / uint16 [num_blocks, Hkv, 128, 256]
    q: np.ndarray                  # uint16 bf16 bits / uint8 e4m3 codes [rows, Hq, 128]
    topk: np.ndarray | None        # int32 [rows, Hkv, k] logical block ids, -1 pad
    sm_scale: float = HEAD_DIM ** -0.5
    k_scale: float = 1.0
    v_scale: float = 1.0
    q_dtype: str = Q_BF16
    q_scale: float = 1.0
    max_blocks: int = 0            # ceil(max seq / 128)
    replicas: list = field(default_factory=list)   # [(q, topk)] extra sets
    notes: str = ""

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def real_rows(self) -> int:
        return self.batch * self.dql

    def positions(self) -> np.ndarray:
        """pos[t] for the real token rows (0-based absolute position)."""
        r = np.arange(self.real_rows) // self.dql
        loc = np.arange(self.real_rows) % self.dql
        return self.seq_lens[r].astype(np.int64) - self.dql + loc


# ---------------------------------------------------------------------------
# page tables and index lists
# ---------------------------------------------------------------------------

def pages_for(seq_len: int) -> int:
    return (int(seq_len) + PAGE - 1) // PAGE


def paged_layout(rng: np.random.Generator, seq_lens, spare_pages: int = 0,
                 fill_page: int | None = None):
    """Block table over a shuffled physical pool (like ``_make_paged_layout``).

    Returns (block_table int32 [B, max_pages], num_pages, spare_ids).  Spare
    pages are extra physical pages no request owns; unused table entries point
    at ``fill_page`` (default: the first spare page if any, else 0).
    """
    per = [pages_for(s) for s in seq_lens]
    used = int(sum(per))
    total = used + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    owned, spare = perm[:used], perm[used:]
    if fill_page is None:
        fill_page = int(spare[0]) if spare_pages else 0
    bt = np.full((len(seq_lens), max(per)), fill_page, dtype=np.int32)
    off = 0
    for r, n in enumerate(per):
        bt[r, :n] = owned[off:off + n]
        off += n
    return bt, total, spare


def last_visible_block(pos: int) -> int:
    return int(pos) // PAGE


def pick_uniform(rng: np.random.Generator, last: int, k: int) -> np.ndarray:
    """k distinct blocks from [0, last], always including ``last``, shuffled."""
    n = last + 1
    if n <= k:
        sel = np.arange(n, dtype=np.int64)
    else:
        others = rng.choice(last, size=k - 1, replace=False)
        sel = np.concatenate([others, [last]])
    return rng.permutation(sel).astype(np.int32)


def pick_zipf_recent(rng: np.random.Generator, last: int, k: int) -> np.ndarray:
    """``last`` plus k-1 distinct earlier blocks with weight 1/(last-b)."""
    if last + 1 <= k:
        return rng.permutation(np.arange(last + 1)).astype(np.int32)
    d = np.arange(last, 0, -1, dtype=np.float64)   # distance of block b=0..last-1
    w = 1.0 / d
    w /= w.sum()
    others = rng.choice(last, size=k - 1, replace=False, p=w)
    sel = np.concatenate([others, [last]])
    return rng.permutation(sel).astype(np.int32)


def pick_zipf_recent_heads(rng: np.random.Generator, last: int, k: int,
                           num_kv_heads: int) -> np.ndarray:
    """``pick_zipf_recent`` for several kv heads at once, by Gumbel top-k:
    the k-1 largest of log(1/(last-b)) + Gumbel noise over b < last are a draw
    without replacement with weights 1/(last-b).  Returns int32 [heads, k],
    -1 padded."""
    out = np.full((num_kv_heads, k), -1, dtype=np.int32)
    if last + 1 <= k:
        for h in range(num_kv_heads):
            out[h, :last + 1] = rng.permutation(np.arange(last + 1))
        return out
    logw = -np.log(np.arange(last, 0, -1, dtype=np.float64))        # block b = 0..last-1
    key = logw[None, :] + rng.gumbel(size=(num_kv_heads, last))
    others = np.argpartition(-key, k - 2, axis=1)[:, : k - 1]
    sel = np.concatenate([others, np.full((num_kv_heads, 1), last)], axis=1)
    for h in range(num_kv_heads):
        out[h] = rng.permutation(sel[h])
    return out


def pad_row(sel: np.ndarray, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int32)
    out[: len(sel)] = sel[:k]
    return out


def every_visible_topk(seq_lens, num_kv_heads: int, dql: int, k: int) -> np.ndarray:
    """Every block a token can see, ascending, then -1 (the index pattern of
    the vLLM test file's ``_make_topk`` fixture), built from the rule: token
    row ``t = r*dql + l`` sits at ``pos = seq_len - dql + l`` and sees blocks
    ``0 .. pos // 128`` (none when ``pos < 0``), capped at k slots."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    rows = len(seq) * dql
    t = np.arange(rows)
    pos = seq[t // dql] - dql + (t % dql)
    last = np.where(pos >= 0, pos // PAGE, -1)
    slots = np.arange(k)
    sel = np.where(slots[None, :] <= last[:, None], slots[None, :], -1).astype(np.int32)
    return np.ascontiguousarray(np.broadcast_to(sel[:, None, :], (rows, num_kv_heads, k)))


def poison_tail_slots(kv: np.ndarray, block_table, seq_lens, kv_dtype: str) -> None:
    """Write NaN patterns into the slots past seq_len of every last page (a
    4-bit page: NaN block scales and all-ones data for those rows)."""
    bad = FP8_NAN_CODE if kv_dtype in KV_8BIT else BF16_NAN_BITS
    for r, s in enumerate(seq_lens):
        n = pages_for(s)
        used = int(s) - (n - 1) * PAGE
        if used >= PAGE:
            continue
        page = block_table[r, n - 1]
        if kv_dtype == KV_MXFP4:
            slots = kv[page].reshape(kv.shape[1], MXFP4_SLOT_BYTES)
            slots[:, used * (HEAD_DIM // 2):MXFP4_DATA_BYTES] = 0xFF
            slots[:, MXFP4_DATA_BYTES + used * (HEAD_DIM // MXFP4_BLOCK):] = MXFP4_NAN_SCALE
        else:
            kv[page, :, used:, :] = bad


def fill_pages(kv: np.ndarray, pages, kv_dtype: str) -> None:
    bad = FP8_NAN_CODE if kv_dtype in KV_8BIT else BF16_NAN_BITS
    if kv_dtype == KV_MXFP4:
        bad = 0xFF            # -6 data, NaN scales
    for p in pages:
        kv[int(p)] = bad


def make_pool(rng: np.random.Generator, num_pages: int, num_kv_heads: int,
              kv_dtype: str, std: float, chunk_pages: int = 256, k_scale: float = 1.0,
              v_scale: float = 1.0) -> np.ndarray:
    """Packed K|V pool ``(num_pages, Hkv, 128, 256)``; values N(0, std), K
    divided by ``k_scale`` and V by ``v_scale``, encoded.  A 4-bit pool is
    ``(num_pages, 2*Hkv, 128, 68)`` head slots (module docstring).

    One 63-bit pool seed is drawn from ``rng``; page chunk ``i`` is then drawn
    from ``default_rng([pool_seed, i])``, so chunks are independent,
    reproducible one at a time, and generated on several threads.
    """
    fp4 = kv_dtype == KV_MXFP4
    if fp4:
        kv = np.empty((num_pages, 2 * num_kv_heads, PAGE, MXFP4_SLOT_BYTES // PAGE),
                      dtype=np.uint8)
    else:
        dt = np.uint8 if kv_dtype in KV_8BIT else np.uint16
        kv = np.empty((num_pages, num_kv_heads, PAGE, 2 * HEAD_DIM), dtype=dt)
    pool_seed = int(rng.integers(0, 2 ** 63 - 1))

    def fill(i):
        p0 = i * chunk_pages
        p1 = min(num_pages, p0 + chunk_pages)
        crng = np.random.default_rng([pool_seed, i])
        x = _normal_f32(crng, (p1 - p0, num_kv_heads, PAGE, 2 * HEAD_DIM), std)
        if k_scale != 1.0:
            x[..., :HEAD_DIM] /= np.float32(k_scale)
        if v_scale != 1.0:
            x[..., HEAD_DIM:] /= np.float32(v_scale)
        if fp4:
            pack_mxfp4_pages(x, kv[p0:p1])
        else:
            kv[p0:p1] = _encode(x, kv_dtype)

    n_chunks = (num_pages + chunk_pages - 1) // chunk_pages
    workers = max(1, min(8, os.cpu_count() or 1, n_chunks))
    if workers == 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return kv


def make_q(rng: np.random.Generator, rows: int, num_q_heads: int, std: float = 1.0,
           q_dtype: str = Q_BF16, q_scale: float = 1.0):
    """Q ~ N(0, std): bf16 bits, or e4m3fn codes of q / q_scale."""
    x = _normal_f32(rng, (rows, num_q_heads, HEAD_DIM), std)
    if q_dtype == Q_FP8:
        return encode_e4m3fn(x / np.float32(q_scale))
    return encode_bf16(x)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = ("c1_tiny_bf16", "c2_tp4_fp8", "c3_tp1_fp8", "c4_spec_ragged",
                "c5_full_step")
# The c2 shape through the two other input formats: fp8 q with a per-tensor
# q_scale over the fp8 e4m3 cache, and bf16 q over an fp8 e5m2 cache.
# The 4-bit cache on the same shape, with the global scales of the test page's
# NVFP4 decode test (k 0.5, v 2.0), under a bf16 and an fp8 q.
FORMAT_CONFIG_NAMES = ("c2_tp4_fp8q", "c2_tp4_e5m2", "c2_tp4_mxfp4", "c2_tp4_mxfp4_fp8q")
C2_FP8Q_SCALE = 0.5
MXFP4_K_SCALE = 0.5
MXFP4_V_SCALE = 2.0


def _topk_rows(rng, seq_lens, dql, hkv, k, rule, per_head, pad_rows=0):
    rows = len(seq_lens) * dql
    topk = np.full((rows + pad_rows, hkv, k), -1, dtype=np.int32)
    for r, s in enumerate(seq_lens):
        for loc in range(dql):
            t = r * dql + loc
            pos = int(s) - dql + loc
            last = last_visible_block(pos)
            if per_head:
                for h in range(hkv):
                    topk[t, h] = pad_row(rule(r, last), k)
            else:
                topk[t, :] = pad_row(rule(r, last), k)
    return topk


def make_config(name: str, replicas: int = 0, poison: bool = True) -> DecodeCase:
    """Build one of the five named workloads (seeded 1..5)."""
    if name == "c1_tiny_bf16":
        return _make_c1(replicas, poison)
    if name == "c2_tp4_fp8":
        return _make_c2(replicas, poison)
    if name == "c2_tp4_fp8q":
        return _make_c2(replicas, poison, q_dtype=Q_FP8, q_scale=C2_FP8Q_SCALE,
                        name=name)
    if name == "c2_tp4_e5m2":
        return _make_c2(replicas, poison, kv_dtype=KV_E5M2, name=name)
    if name == "c2_tp4_mxfp4":
        return _make_c2(replicas, poison, kv_dtype=KV_MXFP4, name=name,
                        k_scale=MXFP4_K_SCALE, v_scale=MXFP4_V_SCALE)
    if name == "c2_tp4_mxfp4_fp8q":
        return _make_c2(replicas, poison, kv_dtype=KV_MXFP4, name=name, q_dtype=Q_FP8,
                        q_scale=C2_FP8Q_SCALE, k_scale=MXFP4_K_SCALE,
                        v_scale=MXFP4_V_SCALE)
    if name == "c3_tp1_fp8":
        return _make_c3(replicas, poison)
    if name == "c4_spec_ragged":
        return _make_c4(replicas, poison)
    if name == "c5_full_step":
        return _make_c5(replicas, poison)
    raise KeyError(name)


def _make_c1(replicas: int, poison: bool) -> DecodeCase:
    rng = np.random.default_rng(1)
    seq = np.array([512, 1000], dtype=np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=4)
    assert total == 16
    kv = make_pool(rng, total, 1, KV_BF16, 1.0)
    if poison:
        fill_pages(kv, spare, KV_BF16)
        poison_tail_slots(kv, bt, seq, KV_BF16)

    def one(rng_):
        q = make_q(rng_, 2, 16)
        topk = _topk_rows(rng_, seq, 1, 1, 4,
                          lambda r, last: pick_uniform(rng_, last, 4), False)
        return q, topk

    q, topk = one(rng)
    reps = [one(rng) for _ in range(replicas)]
    return DecodeCase("c1_tiny_bf16", 1, 2, 1, 2, 16, 1, 4, KV_BF16, seq, bt, kv,
                      q, topk, max_blocks=int(bt.shape[1]), replicas=reps)


def _make_c2(replicas: int, poison: bool, q_dtype: str = Q_BF16, q_scale: float = 1.0,
             kv_dtype: str = KV_FP8, name: str = "c2_tp4_fp8", k_scale: float = 1.0,
             v_scale: float = 1.0) -> DecodeCase:
    rng = np.random.default_rng(2)
    B, dql, hq, hkv, k = 32, 4, 16, 1, 16
    seq = rng.integers(16384, 65536, size=B, endpoint=True).astype(np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, hkv, kv_dtype, 0.5, k_scale=k_scale, v_scale=v_scale)
    if poison:
        fill_pages(kv, spare, kv_dtype)
        poison_tail_slots(kv, bt, seq, kv_dtype)

    def one(rng_):
        q = make_q(rng_, B * dql, hq, q_dtype=q_dtype, q_scale=q_scale)
        topk = _topk_rows(rng_, seq, dql, hkv, k,
                          lambda r, last: pick_uniform(rng_, last, k), False)
        return q, topk

    q, topk = one(rng)
    reps = [one(rng) for _ in range(replicas)]
    return DecodeCase(name, 2, B, dql, B * dql, hq, hkv, k, kv_dtype, seq, bt,
                      kv, q, topk, q_dtype=q_dtype, q_scale=q_scale, k_scale=k_scale,
                      v_scale=v_scale, max_blocks=int(bt.shape[1]), replicas=reps)


def _make_c3(replicas: int, poison: bool) -> DecodeCase:
    rng = np.random.default_rng(3)
    B, dql, hq, hkv, k = 16, 4, 64, 4, 16
    seq = rng.integers(32768, 131072, size=B, endpoint=True).astype(np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, hkv, KV_FP8, 0.5)
    if poison:
        fill_pages(kv, spare, KV_FP8)
        poison_tail_slots(kv, bt, seq, KV_FP8)

    def one(rng_):
        q = make_q(rng_, B * dql, hq)
        topk = _topk_rows(rng_, seq, dql, hkv, k,
                          lambda r, last: pick_zipf_recent(rng_, last, k), True)
        return q, topk

    q, topk = one(rng)
    reps = [one(rng) for _ in range(replicas)]
    return DecodeCase("c3_tp1_fp8", 3, B, dql, B * dql, hq, hkv, k, KV_FP8, seq, bt,
                      kv, q, topk, max_blocks=int(bt.shape[1]), replicas=reps)


def _make_c4(replicas: int, poison: bool) -> DecodeCase:
    rng = np.random.default_rng(4)
    B, dql, hq, hkv, k, pad = 16, 32, 64, 4, 16, 4
    long_ids = np.sort(rng.permutation(B)[: B // 2])
    seq = np.empty(B, dtype=np.int32)
    for r in range(B):
        seq[r] = 131072 if r in long_ids else int(rng.integers(200, 1900, endpoint=True))
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, hkv, KV_FP8, 0.5)
    if poison:
        fill_pages(kv, spare, KV_FP8)
        poison_tail_slots(kv, bt, seq, KV_FP8)
    is_long = np.isin(np.arange(B), long_ids)

    def rule(rng_):
        def f(r, last):
            if is_long[r]:
                return pick_zipf_recent(rng_, last, k)
            return rng_.permutation(np.arange(last + 1)).astype(np.int32)
        return f

    def one(rng_):
        q = make_q(rng_, B * dql + pad, hq)
        topk = _topk_rows(rng_, seq, dql, hkv, k, rule(rng_), True, pad_rows=pad)
        return q, topk

    q, topk = one(rng)
    reps = [one(rng) for _ in range(replicas)]
    return DecodeCase("c4_spec_ragged", 4, B, dql, B * dql + pad, hq, hkv, k, KV_FP8,
                      seq, bt, kv, q, topk, max_blocks=int(bt.shape[1]), replicas=reps,
                      notes="rows 512..515 are padding rows")


def make_dense_config(name: str, replicas: int = 0, poison: bool = True) -> DecodeCase:
    """Dense decode (every visible block; M3's first layers): the TP1 decode
    shape -- B=16, dql=4, 64/4 heads, fp8 e4m3, seq U[32768, 131072] -- with
    no top-k (seed 7)."""
    if name != "d1_dense_tp1":
        raise KeyError(name)
    rng = np.random.default_rng(7)
    B, dql, hq, hkv = 16, 4, 64, 4
    seq = rng.integers(32768, 131072, size=B, endpoint=True).astype(np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, hkv, KV_FP8, 0.5)
    if poison:
        fill_pages(kv, spare, KV_FP8)
        poison_tail_slots(kv, bt, seq, KV_FP8)
    q = make_q(rng, B * dql, hq)
    reps = [(make_q(rng, B * dql, hq), None) for _ in range(replicas)]
    return DecodeCase(name, 7, B, dql, B * dql, hq, hkv, 0, KV_FP8, seq, bt, kv, q, None,
                      max_blocks=int(bt.shape[1]), replicas=reps,
                      notes="dense: every visible block, no top-k")


DENSE_CONFIG_NAMES = ("d1_dense_tp1",)


def c5_seq_lens(rng: np.random.Generator, B: int = 64) -> np.ndarray:
    mu = math.log(math.sqrt(8192.0 * 262144.0))
    sigma = math.log(32.0) / 4.0
    s = np.exp(rng.normal(mu, sigma, size=B))
    return np.clip(np.rint(s), 8192, 262144).astype(np.int32)


def _make_c5(replicas: int, poison: bool) -> DecodeCase:
    rng = np.random.default_rng(5)
    B, dql, hq, hkv, k = 64, 1, 64, 4, 16
    seq = c5_seq_lens(rng, B)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, hkv, KV_FP8, 0.5)
    if poison:
        fill_pages(kv, spare, KV_FP8)
        poison_tail_slots(kv, bt, seq, KV_FP8)
    q = make_q(rng, B, hq)
    reps = [(make_q(rng, B, hq), None) for _ in range(replicas)]
    return DecodeCase("c5_full_step", 5, B, dql, B, hq, hkv, k, KV_FP8, seq, bt, kv, q,
                      None, max_blocks=int(bt.shape[1]), replicas=reps,
                      notes="top-k comes from the block-max scorer and selector")


# ---------------------------------------------------------------------------
# small cases for parity and oracle pins
# ---------------------------------------------------------------------------

def make_p3_case(num_q_heads: int, num_kv_heads: int, pairs: int, dql: int,
                 seq_pattern=(257, 513), seed: int = 0, kv_dtype: str = KV_FP8,
                 std: float = 0.25, topk_k: int = 16, poison: bool = True,
                 q_dtype: str = Q_BF16, q_scale: float = 1.0, k_scale: float = 1.0,
                 v_scale: float = 1.0) -> DecodeCase:
    """The test page's parity shape: seq_lens = pattern * pairs, every visible
    page selected (``_make_topk``), K and V ~ N(0, std) encoded, Q ~ N(0,1)."""
    rng = np.random.default_rng(1000 + seed)
    seq = np.array(list(seq_pattern) * pairs, dtype=np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, num_kv_heads, kv_dtype, std, k_scale=k_scale, v_scale=v_scale)
    if poison:
        fill_pages(kv, spare, kv_dtype)
        poison_tail_slots(kv, bt, seq, kv_dtype)
    rows = len(seq) * dql
    q = make_q(rng, rows, num_q_heads, q_dtype=q_dtype, q_scale=q_scale)
    topk = every_visible_topk(seq, num_kv_heads, dql, topk_k)
    return DecodeCase(f"p3_h{num_q_heads}_{num_kv_heads}_pairs{pairs}_dql{dql}", seed,
                      len(seq), dql, rows, num_q_heads, num_kv_heads, topk_k, kv_dtype,
                      seq, bt, kv, q, topk, q_dtype=q_dtype, q_scale=q_scale,
                      k_scale=k_scale, v_scale=v_scale, max_blocks=int(bt.shape[1]))


def make_random_case(seed: int, batch: int, dql: int, num_q_heads: int,
                     num_kv_heads: int, topk_k: int, seq_lo: int, seq_hi: int,
                     kv_dtype: str = KV_FP8, std: float = 0.5, pad_rows: int = 0,
                     per_head: bool = True, rule: str = "uniform",
                     neg_frac: float = 0.0, poison: bool = True,
                     stride_extra: int = 0, q_dtype: str = Q_BF16,
                     q_scale: float = 1.0, k_scale: float = 1.0,
                     v_scale: float = 1.0) -> DecodeCase:
    """A generic seeded case: uniform seq lens, random distinct blocks that
    include each token's causal last block, optional extra -1 entries."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(seq_lo, seq_hi, size=batch, endpoint=True).astype(np.int32)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    if stride_extra:
        bt = np.concatenate(
            [bt, np.full((batch, stride_extra), bt[0, 0], dtype=np.int32)], axis=1)
    kv = make_pool(rng, total, num_kv_heads, kv_dtype, std, k_scale=k_scale, v_scale=v_scale)
    if poison:
        fill_pages(kv, spare, kv_dtype)
        poison_tail_slots(kv, bt, seq, kv_dtype)
    rows = batch * dql
    q = make_q(rng, rows + pad_rows, num_q_heads, q_dtype=q_dtype, q_scale=q_scale)
    pick = pick_uniform if rule == "uniform" else pick_zipf_recent
    topk = _topk_rows(rng, seq, dql, num_kv_heads, topk_k,
                      lambda r, last: pick(rng, last, topk_k), per_head,
                      pad_rows=pad_rows)
    if neg_frac > 0:
        mask = rng.random(topk.shape) < neg_frac
        topk[mask] = -1
    return DecodeCase(f"rand_s{seed}", seed, batch, dql, rows + pad_rows, num_q_heads,
                      num_kv_heads, topk_k, kv_dtype, seq, bt, kv, q, topk,
                      q_dtype=q_dtype, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale,
                      max_blocks=int(bt.shape[1]))


@dataclass
class PrefillCase:
    """One ragged prefill step: request r owns q rows cu[r]..cu[r+1]-1 and its
    local token i sits at context_lens[r] + i."""

    name: str
    seed: int
    q_lens: np.ndarray             # int32 [batch]
    seq_lens: np.ndarray           # int32 [batch], context + q_len
    context_lens: np.ndarray       # int32 [batch]
    cu_seqlens_q: np.ndarray       # int32 [batch + 1]
    num_token_rows: int            # >= cu[-1]; rows past it are padding
    num_q_heads: int
    num_kv_heads: int
    topk_k: int
    kv_dtype: str
    block_table: np.ndarray
    kv: np.ndarray
    q: np.ndarray
    topk: np.ndarray               # int32 [rows, Hkv, k]
    sm_scale: float = HEAD_DIM ** -0.5
    k_scale: float = 1.0
    v_scale: float = 1.0
    q_dtype: str = Q_BF16
    q_scale: float = 1.0
    max_blocks: int = 0
    replicas: list = field(default_factory=list)   # [(q, topk)] extra sets

    @property
    def batch(self) -> int:
        return int(len(self.q_lens))

    @property
    def real_rows(self) -> int:
        return int(self.cu_seqlens_q[-1])

    def positions(self) -> np.ndarray:
        """pos[t] for the real token rows."""
        r = np.repeat(np.arange(self.batch), self.q_lens)
        local = np.arange(self.real_rows) - self.cu_seqlens_q[r]
        return self.context_lens[r].astype(np.int64) + local


def make_prefill_case(seed: int, q_lens, seq_lens, num_q_heads: int, num_kv_heads: int,
                      topk_k: int = 16, kv_dtype: str = KV_FP8, q_dtype: str = Q_BF16,
                      q_scale: float = 1.0, rule: str = "every_visible", std: float = 0.25,
                      pad_rows: int = 0, replicas: int = 0, poison: bool = True,
                      name: str = "", k_scale: float = 1.0,
                      v_scale: float = 1.0) -> PrefillCase:
    """A seeded ragged prefill step.  rule "every_visible" selects blocks
    0..last for each token (the test page's prefill test, which needs
    last < topk_k); "zipf" picks topk_k distinct blocks per (token, kv head)
    with the recent bias, always including the token's own block."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    seq = np.asarray(seq_lens, dtype=np.int32)
    ctx = (seq - q_lens).astype(np.int32)
    assert np.all(ctx >= 0)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    bt, total, spare = paged_layout(rng, seq, spare_pages=1)
    kv = make_pool(rng, total, num_kv_heads, kv_dtype, std, k_scale=k_scale, v_scale=v_scale)
    if poison:
        fill_pages(kv, spare, kv_dtype)
        poison_tail_slots(kv, bt, seq, kv_dtype)
    rows = int(cu[-1]) + pad_rows

    def one(rng_):
        q = make_q(rng_, rows, num_q_heads, q_dtype=q_dtype, q_scale=q_scale)
        topk = np.full((rows, num_kv_heads, topk_k), -1, dtype=np.int32)
        for r in range(len(q_lens)):
            for i in range(int(q_lens[r])):
                t = int(cu[r]) + i
                last = last_visible_block(int(ctx[r]) + i)
                if rule == "every_visible":
                    assert last < topk_k
                    topk[t, :, :last + 1] = np.arange(last + 1, dtype=np.int32)
                else:
                    topk[t] = pick_zipf_recent_heads(rng_, last, topk_k, num_kv_heads)
        return q, topk

    q, topk = one(rng)
    reps = [one(rng) for _ in range(replicas)]
    return PrefillCase(name or f"prefill_s{seed}", seed, q_lens, seq, ctx, cu, rows,
                       num_q_heads, num_kv_heads, topk_k, kv_dtype, bt, kv, q, topk,
                       q_dtype=q_dtype, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale,
                       max_blocks=int(bt.shape[1]), replicas=reps)


PREFILL_CONFIG_NAMES = ("pf1_chunked_prefill",)


def make_prefill_config(name: str, replicas: int = 0, poison: bool = True) -> PrefillCase:
    """Chunked prefill: 4 requests each adding a 1024-token chunk after a
    cached context of U[16384, 65536] tokens, 64/4 heads, fp8 e4m3 cache,
    top-16 per (token, kv head) with the recent bias and the token's own
    block (the shape the pages' prefill path serves; they print no prefill
    benchmark)."""
    if name != "pf1_chunked_prefill":
        raise KeyError(name)
    rng = np.random.default_rng(6)
    B, chunk = 4, 1024
    ctx = rng.integers(16384, 65536, size=B, endpoint=True).astype(np.int32)
    q_lens = np.full(B, chunk, dtype=np.int32)
    return make_prefill_case(int(rng.integers(0, 2 ** 31 - 1)), q_lens, ctx + q_lens, 64, 4,
                             topk_k=16, kv_dtype=KV_FP8, rule="zipf", std=0.5,
                             replicas=replicas, poison=poison, name=name)


def make_scores(seed: int, num_kv_heads: int, max_blocks: int, rows: int, seq_lens,
                dql: int, tie_frac: float = 0.0) -> np.ndarray:
    """fp32 score buffer [Hkv, max_blocks, rows] for selector tests: N(0,1)
    values for causally visible blocks, -inf elsewhere; optionally with
    planted exact ties (copied values)."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((num_kv_heads, max_blocks, rows)).astype(np.float32)
    for r, sl in enumerate(seq_lens):
        for loc in range(dql):
            t = r * dql + loc
            pos = int(sl) - dql + loc
            nvis = pos // PAGE + 1 if pos >= 0 else 0
            s[:, nvis:, t] = -np.inf
    if tie_frac > 0:
        for h in range(num_kv_heads):
            for t in range(rows):
                fin = np.nonzero(np.isfinite(s[h, :, t]))[0]
                if len(fin) < 2:
                    continue
                n = max(1, int(tie_frac * len(fin)))
                src = rng.choice(fin, size=n)
                dst = rng.choice(fin, size=n)
                s[h, dst, t] = s[h, src, t]
    return s
