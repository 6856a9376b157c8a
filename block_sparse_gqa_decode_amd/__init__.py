"""Block-sparse GQA decode attention for MI355X (gfx950).

Python binding over ``libmsa_decode.so`` (C ABI: ``include/msa_sparse_decode.h``).
This module only marshals arguments: every step of the decode path runs in the
library's HIP kernels, and there is no fallback.  If the library is not built,
every call raises.

Entry points carry the C names:

* ``msa_sparse_decode_plan``  -- validate a static shape, build a plan (with its
  persistent split-K arena); ``PlanCache`` keys plans like the plan cache of the
  vLLM API page ``vllm.models.minimax_m3.nvidia.msa_cutlass_sparse_decode``
  (``MSACutlassDecodePlanCache.prepare``).
* ``msa_sparse_decode_run``   -- one sparse decode step (the attend).
* ``msa_sparse_prefill_plan`` / ``msa_sparse_prefill_run`` -- the same attend
  over ragged prefill chunks (``cu_seqlens_q``, ``context_lens``).
* ``msa_block_score_topk``    -- indexer block-max scores, then the top-k.
* ``msa_topk_select``         -- the top-k selector alone.
* ``msa_fp8_e4m3_to_bf16`` / ``msa_fp8_e5m2_to_bf16`` -- the in-register fp8
  conversions, as a check.
* ``msa_mxfp4_to_bf16``       -- a 4-bit (MXFP4 head-slot) cache dequantized to
  packed bf16 K|V rows with the attend's own conversion.

Tensor checks follow ``MSACutlassDecodePlanCache.prepare`` (contiguous int32
block table with one row per request, contiguous int32 sequence lengths on the
same device) and the backend contract of the vLLM API page
``vllm.models.minimax_m3.common.sparse_attention`` (head size 128, page size
128, bf16, fp8 e4m3 or fp8 e5m2 KV in a packed ``(num_blocks, Hkv, 128, 256)``
cache).  A 4-bit cache (``KV_MXFP4``) is a ``uint8 (num_blocks, 2*Hkv, 128,
68)`` tensor of head slots -- slot 2h holds K of kv head h, slot 2h+1 its V,
each as 128 rows of 64 e2m1 code bytes then 128 rows of 4 E8M0 scales (the
NVFP4 head-slot page of vLLM's MSA test file, with OCP MX blocks of 32).  q is
bf16, or fp8 e4m3 codes with a per-tensor ``q_scale`` (the ``query_fp8`` /
``q_scale_float`` arguments of ``msa_cutlass_sparse_decode``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MsaError", "MsaInvalidArgument", "MsaUnsupported", "DecodePlan", "PlanCache",
    "msa_sparse_decode_plan", "msa_sparse_decode_run", "msa_sparse_decode_attend",
    "msa_sparse_decode_merge", "msa_sparse_decode_run_noalloc", "msa_sparse_decode_select_run",
    "msa_block_score_topk", "msa_sparse_prefill_plan",
    "msa_sparse_prefill_run",
    "msa_topk_select", "msa_fp8_e4m3_to_bf16", "msa_fp8_e5m2_to_bf16", "msa_mxfp4_to_bf16",
    "msa_probe_read_runs",
    "library_path", "load_library", "KV_BF16", "KV_FP8_E4M3", "KV_FP8_E5M2", "KV_MXFP4",
    "Q_BF16", "Q_FP8_E4M3",
    "PAGE_SIZE", "HEAD_DIM", "ABI_VERSION",
]

ABI_VERSION = 7
PAGE_SIZE = 128
HEAD_DIM = 128
KV_BF16 = 0
KV_FP8_E4M3 = 1
KV_FP8_E5M2 = 2
KV_MXFP4 = 3
MXFP4_SLOT_ROW_BYTES = 68   # a slot's 8704 bytes viewed as 128 x 68
Q_BF16 = 0
Q_FP8_E4M3 = 1

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_DEVICE = -3
MSA_ERR_OUT_OF_MEMORY = -4

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmsa_decode.so"


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[msa status {status}] {message}")
        self.status = status


class MsaInvalidArgument(MsaError, ValueError):
    pass


class MsaUnsupported(MsaError, NotImplementedError):
    pass


class _Shape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "decode_query_len", "num_token_rows", "page_table_stride",
        "num_q_heads", "num_kv_heads", "page_size", "head_dim", "topk_blocks",
        "kv_dtype", "num_splits", "q_dtype", "tile_rows")]


class _PrefillShape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_prefills", "num_token_rows", "page_table_stride", "num_q_heads",
        "num_kv_heads", "page_size", "head_dim", "topk_blocks", "kv_dtype", "q_dtype",
        "num_splits", "tile_rows")]


_I64x4 = ctypes.c_int64 * 4
_I64x3 = ctypes.c_int64 * 3
_LIB = None


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library():
    """Load the built HIP library (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python -m block_sparse_gqa_decode_amd.build_lib`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    pi64 = ctypes.POINTER(ctypes.c_int64)
    sig = {
        "msa_sparse_decode_plan": (i32, [ctypes.POINTER(_Shape), ctypes.c_int,
                                         ctypes.POINTER(vp)]),
        "msa_sparse_decode_plan_destroy": (i32, [vp]),
        "msa_sparse_decode_plan_info": (i32, [vp, ctypes.POINTER(i32), ctypes.POINTER(i64),
                                              ctypes.POINTER(_Shape)]),
        "msa_sparse_decode_run": (i32, [vp, vp, vp, pi64, i64, f32, f32, f32, vp, vp, vp,
                                        pi64, vp, f32, vp]),
        "msa_sparse_decode_attend": (i32, [vp, vp, vp, pi64, i64, f32, f32, f32, vp, vp,
                                           vp, pi64, vp, f32, vp]),
        "msa_sparse_decode_merge": (i32, [vp, vp, f32, vp]),
        "msa_sparse_decode_select_run": (i32, [vp, vp, vp, pi64, i64, f32, f32, f32, vp, vp,
                                               vp, pi64, i32, vp, vp, f32, vp]),
        "msa_sparse_decode_run_noalloc": (i32, [ctypes.POINTER(_Shape), ctypes.c_int, vp, vp,
                                                pi64, i64, f32, f32, f32, vp, vp, vp, pi64, vp,
                                                f32, vp]),
        "msa_sparse_prefill_plan": (i32, [ctypes.POINTER(_PrefillShape), ctypes.c_int,
                                          ctypes.POINTER(vp)]),
        "msa_sparse_prefill_run": (i32, [vp, vp, vp, pi64, i64, f32, f32, f32, vp, vp, vp,
                                         vp, pi64, vp, f32, vp]),
        "msa_block_score_topk": (i32, [ctypes.POINTER(_Shape), vp, vp, pi64, i64, f32, f32,
                                       vp, vp, i32, vp, pi64, vp, i32, vp]),
        "msa_topk_select": (i32, [vp, pi64, i32, i32, i32, vp, i32, vp]),
        "msa_fp8_e4m3_to_bf16": (i32, [vp, vp, i64, vp]),
        "msa_fp8_e5m2_to_bf16": (i32, [vp, vp, i64, vp]),
        "msa_mxfp4_to_bf16": (i32, [vp, pi64, i64, i32, vp, vp]),
        "msa_probe_read_runs": (i32, [vp, i64, vp, vp, i32, vp, i32, vp, vp]),
        "msa_last_error": (ctypes.c_char_p, []),
        "msa_abi_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.msa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.msa_abi_version()}, the binding "
                           f"expects {ABI_VERSION}: rebuild the library")
    _LIB = lib
    return lib


def _check(status: int):
    if status == MSA_OK:
        return
    msg = load_library().msa_last_error().decode(errors="replace")
    if status == MSA_ERR_INVALID_ARG:
        raise MsaInvalidArgument(status, msg)
    if status == MSA_ERR_UNSUPPORTED:
        raise MsaUnsupported(status, msg)
    raise MsaError(status, msg)


def _stream_handle(stream, device) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _kv_dtype_of(kv: torch.Tensor, declared: Optional[int] = None) -> int:
    """The KV format of a cache tensor.  ``uint8`` holds either fp8 format or
    4-bit head slots and takes ``declared`` (default e4m3); typed fp8 tensors
    must agree with it."""
    if kv.dtype == torch.uint8:
        return KV_FP8_E4M3 if declared is None else declared
    found = {torch.float8_e4m3fn: KV_FP8_E4M3, torch.float8_e5m2: KV_FP8_E5M2,
             torch.bfloat16: KV_BF16}.get(kv.dtype)
    if found is None:
        raise ValueError(f"unsupported kv cache dtype {kv.dtype}: expected bfloat16, "
                         "float8_e4m3fn, float8_e5m2 or uint8")
    if declared is not None and found != declared:
        raise ValueError("kv_cache dtype does not match the declared kv_dtype")
    return found


def _q_dtype_of(q: torch.Tensor) -> int:
    if q.dtype == torch.bfloat16:
        return Q_BF16
    if q.dtype in (torch.float8_e4m3fn, torch.uint8):
        return Q_FP8_E4M3
    raise ValueError(f"unsupported q dtype {q.dtype}: expected bfloat16 or float8_e4m3fn")


def _check_kv(kv: torch.Tensor, num_kv_heads: int, kv_dtype: Optional[int] = None):
    if kv.device.type != "cuda":
        raise ValueError("kv_cache must be a device tensor")
    if kv_dtype == KV_MXFP4:
        if kv.dtype != torch.uint8 or kv.dim() != 4 or kv.shape[1] != 2 * num_kv_heads \
                or kv.shape[2] != PAGE_SIZE or kv.shape[3] != MXFP4_SLOT_ROW_BYTES:
            raise ValueError(f"an MXFP4 kv_cache must be uint8 (num_blocks, "
                             f"{2 * num_kv_heads}, 128, 68), got {kv.dtype} {tuple(kv.shape)}")
        if kv.stride(3) != 1 or kv.stride(2) != MXFP4_SLOT_ROW_BYTES:
            raise ValueError("each MXFP4 head slot must be one contiguous 8704-byte run")
        return
    if kv.dim() != 4 or kv.shape[1] != num_kv_heads or kv.shape[2] != PAGE_SIZE \
            or kv.shape[3] != 2 * HEAD_DIM:
        raise ValueError(f"kv_cache must be logically (num_blocks, {num_kv_heads}, 128, 256), "
                         f"got {tuple(kv.shape)}")
    if kv.stride(3) != 1:
        raise ValueError("kv_cache last dimension must be contiguous")


def _kv_strides(kv: torch.Tensor, kv_dtype: int):
    """kv_strides for the C ABI: element strides, or for 4-bit head slots the
    byte strides (page, head = two slots, K slot -> V slot, 1)."""
    if kv_dtype == KV_MXFP4:
        return _I64x4(kv.stride(0), 2 * kv.stride(1), kv.stride(1), 1)
    return _I64x4(*kv.stride())


def _check_tables(block_table: torch.Tensor, seq_lens: torch.Tensor, batch: int):
    if (block_table.device.type != "cuda" or block_table.dtype != torch.int32
            or not block_table.is_contiguous() or block_table.dim() != 2
            or block_table.shape[0] != batch):
        raise ValueError("MSA sparse decode requires a contiguous device int32 block "
                         "table with one row per request")
    if (seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous()
            or seq_lens.device != block_table.device or seq_lens.shape != (batch,)):
        raise ValueError("MSA sparse decode requires contiguous device int32 sequence "
                         "lengths on the block table device")


def _check_q(q: torch.Tensor, name: str, rows: int, hq: int, q_dtype: int = Q_BF16):
    ok_dtype = q.dtype == torch.bfloat16 if q_dtype == Q_BF16 else \
        q.dtype in (torch.float8_e4m3fn, torch.uint8)
    if q.device.type != "cuda" or not ok_dtype or not q.is_contiguous():
        kind = "bfloat16" if q_dtype == Q_BF16 else "float8_e4m3fn (or uint8 codes)"
        raise ValueError(f"{name} must be a contiguous device {kind} tensor")
    if tuple(q.shape) != (rows, hq, HEAD_DIM):
        raise ValueError(f"{name} must have shape ({rows}, {hq}, {HEAD_DIM}), "
                         f"got {tuple(q.shape)}")


class DecodePlan:
    """A validated static shape plus the library plan (owns the split-K arena)."""

    def __init__(self, handle: int, device: int):
        self._handle = ctypes.c_void_p(handle)
        self.device = device
        splits = ctypes.c_int32()
        arena = ctypes.c_int64()
        shape = _Shape()
        _check(load_library().msa_sparse_decode_plan_info(
            self._handle, ctypes.byref(splits), ctypes.byref(arena), ctypes.byref(shape)))
        self.batch = shape.batch
        self.decode_query_len = shape.decode_query_len   # 0 for a prefill plan
        self.prefill = shape.decode_query_len == 0
        self.num_token_rows = shape.num_token_rows
        self.page_table_stride = shape.page_table_stride
        self.num_q_heads = shape.num_q_heads
        self.num_kv_heads = shape.num_kv_heads
        self.topk_blocks = shape.topk_blocks
        self.kv_dtype = shape.kv_dtype
        self.q_dtype = shape.q_dtype
        self.tile_rows = shape.tile_rows
        self.dense = shape.topk_blocks == 0
        self.num_splits = splits.value
        self.arena_bytes = arena.value
        # Single-row plans with 2..4 splits combine them inside the attend
        # (msa_sparse_decode_attend / _merge in the C header).
        self.merges_in_attend = self.tile_rows == 1 and 2 <= self.num_splits <= 4

    @property
    def handle(self):
        return self._handle

    def close(self):
        if self._handle is not None and self._handle.value:
            _check(load_library().msa_sparse_decode_plan_destroy(self._handle))
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def msa_sparse_decode_plan(batch: int, decode_query_len: int, *, num_q_heads: int,
                           num_kv_heads: int, page_table_stride: int, topk_blocks: int,
                           kv_dtype: int, num_token_rows: int = 0, num_splits: int = 0,
                           page_size: int = PAGE_SIZE, head_dim: int = HEAD_DIM,
                           q_dtype: int = Q_BF16, tile_rows: int = 0,
                           device=None) -> DecodePlan:
    """topk_blocks = 0 plans dense decode (every visible block; run with
    topk=None).  tile_rows: 0 = the plan's choice, 1 = one token row per
    workgroup, 2 / 4 = multi-row tiles."""
    lib = load_library()
    shape = _Shape(batch, decode_query_len, num_token_rows, page_table_stride, num_q_heads,
                   num_kv_heads, page_size, head_dim, topk_blocks, kv_dtype, num_splits,
                   q_dtype, tile_rows)
    if device is None:
        dev = torch.cuda.current_device() if torch.cuda.is_available() else 0
    elif isinstance(device, int):
        dev = device
    else:
        dev = torch.device(device).index
        if dev is None:
            dev = torch.cuda.current_device()
    handle = ctypes.c_void_p()
    _check(lib.msa_sparse_decode_plan(ctypes.byref(shape), int(dev), ctypes.byref(handle)))
    return DecodePlan(handle.value, int(dev))


def _device_index(device) -> int:
    if device is None:
        return torch.cuda.current_device() if torch.cuda.is_available() else 0
    if isinstance(device, int):
        return device
    dev = torch.device(device).index
    return torch.cuda.current_device() if dev is None else dev


def msa_sparse_prefill_plan(num_prefills: int, num_token_rows: int, *, num_q_heads: int,
                            num_kv_heads: int, page_table_stride: int, topk_blocks: int,
                            kv_dtype: int, q_dtype: int = Q_BF16, num_splits: int = 0,
                            page_size: int = PAGE_SIZE, head_dim: int = HEAD_DIM,
                            tile_rows: int = 0, device=None) -> DecodePlan:
    """A plan for ragged prefill chunks over ``num_token_rows`` q rows."""
    lib = load_library()
    shape = _PrefillShape(num_prefills, num_token_rows, page_table_stride, num_q_heads,
                          num_kv_heads, page_size, head_dim, topk_blocks, kv_dtype, q_dtype,
                          num_splits, tile_rows)
    dev = _device_index(device)
    handle = ctypes.c_void_p()
    _check(lib.msa_sparse_prefill_plan(ctypes.byref(shape), int(dev), ctypes.byref(handle)))
    return DecodePlan(handle.value, int(dev))


def msa_sparse_prefill_run(plan: DecodePlan, q: torch.Tensor, kv_cache: torch.Tensor,
                           block_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                           context_lens: torch.Tensor, topk: torch.Tensor, out: torch.Tensor,
                           *, sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                           q_scale: float = 1.0, stream=None) -> None:
    """out[t, j] for ragged prefill chunks: row t of request r (cu[r] <= t <
    cu[r+1]) attends as a decode token at context_lens[r] + t - cu[r]."""
    if not plan.prefill:
        raise ValueError("msa_sparse_prefill_run needs a prefill plan")
    n = plan.batch
    if (cu_seqlens_q.dtype != torch.int32 or not cu_seqlens_q.is_contiguous()
            or tuple(cu_seqlens_q.shape) != (n + 1,)):
        raise ValueError(f"cu_seqlens_q must be contiguous int32 [{n + 1}]")
    if (context_lens.dtype != torch.int32 or not context_lens.is_contiguous()
            or tuple(context_lens.shape) != (n,)):
        raise ValueError(f"context_lens must be contiguous int32 [{n}]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("context_lens", context_lens)):
        if t.device != block_table.device:
            raise ValueError(f"{name} is not on the block table device")
    head = _run_args(plan, q, kv_cache, block_table, context_lens, topk, out, tables=False)
    if (block_table.device.type != "cuda" or block_table.dtype != torch.int32
            or not block_table.is_contiguous() or block_table.dim() != 2
            or block_table.shape[0] != n):
        raise ValueError("MSA sparse prefill requires a contiguous device int32 block "
                         "table with one row per request")
    _check(load_library().msa_sparse_prefill_run(
        *head, float(q_scale), float(k_scale), float(v_scale), block_table.data_ptr(),
        cu_seqlens_q.data_ptr(), context_lens.data_ptr(), topk.data_ptr(),
        _I64x3(*topk.stride()), out.data_ptr(), float(sm_scale),
        _stream_handle(stream, q.device)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _strides3(t: Optional[torch.Tensor]):
    return None if t is None else _I64x3(*t.stride())


def _run_args(plan, q, kv_cache, block_table, seq_lens, topk, out, tables=True,
              selects=False):
    rows = plan.num_token_rows
    _check_q(q, "q", rows, plan.num_q_heads, plan.q_dtype)
    _check_q(out, "out", rows, plan.num_q_heads)
    _kv_dtype_of(kv_cache, plan.kv_dtype)
    _check_kv(kv_cache, plan.num_kv_heads, plan.kv_dtype)
    if tables:
        _check_tables(block_table, seq_lens, plan.batch)
    if block_table.stride(0) != plan.page_table_stride:
        raise ValueError("block_table row stride does not match the plan")
    if selects:
        if plan.dense:
            raise ValueError("a dense plan attends every visible block: nothing to select")
    elif plan.dense:
        if topk is not None:
            raise ValueError("a dense plan attends every visible block: pass topk=None")
    elif (topk is None or topk.dtype != torch.int32 or topk.dim() != 3
            or tuple(topk.shape) != (rows, plan.num_kv_heads, plan.topk_blocks)):
        raise ValueError(f"topk must be int32 [{rows}, {plan.num_kv_heads}, "
                         f"{plan.topk_blocks}], got "
                         f"{None if topk is None else (topk.dtype, tuple(topk.shape))}")
    for name, t in (("kv_cache", kv_cache), ("block_table", block_table), ("topk", topk),
                    ("q", q), ("out", out)):
        if t is None:
            continue
        if t.device != seq_lens.device:
            raise ValueError(f"{name} is not on the sequence-length device")
    return (plan.handle, q.data_ptr(), kv_cache.data_ptr(),
            _kv_strides(kv_cache, plan.kv_dtype), kv_cache.shape[0])


def _require_decode_plan(plan: DecodePlan):
    if plan.prefill:
        raise ValueError("a prefill plan runs through msa_sparse_prefill_run")


def msa_sparse_decode_run(plan: DecodePlan, q: torch.Tensor, kv_cache: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor,
                          topk: Optional[torch.Tensor], out: torch.Tensor, *, sm_scale: float,
                          k_scale: float = 1.0, v_scale: float = 1.0, q_scale: float = 1.0,
                          stream=None) -> None:
    """out[t, j] = sparse causal attention of q[t, j] over the selected pages
    (every visible page with a dense plan and topk=None)."""
    _require_decode_plan(plan)
    head = _run_args(plan, q, kv_cache, block_table, seq_lens, topk, out)
    _check(load_library().msa_sparse_decode_run(
        *head, float(q_scale), float(k_scale), float(v_scale), block_table.data_ptr(), seq_lens.data_ptr(),
        _ptr(topk), _strides3(topk), out.data_ptr(), float(sm_scale),
        _stream_handle(stream, q.device)))


def msa_sparse_decode_select_run(plan: DecodePlan, q: torch.Tensor, kv_cache: torch.Tensor,
                                 block_table: torch.Tensor, seq_lens: torch.Tensor,
                                 score: torch.Tensor, out: torch.Tensor, *, sm_scale: float,
                                 topk_out: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                                 v_scale: float = 1.0, q_scale: float = 1.0,
                                 stream=None) -> None:
    """The attend of msa_sparse_decode_run over the top-k rows that each
    workgroup selects from ``score`` itself (float32 logical [Hkv, max_blocks,
    rows], as msa_block_score_topk fills it); ``topk_out`` (optional, int32
    [rows, Hkv, k]) receives the selection."""
    _require_decode_plan(plan)
    if score.dtype != torch.float32 or score.dim() != 3 or score.device != q.device:
        raise ValueError("score must be a 3-D float32 tensor [Hkv, blocks, rows] on q's device")
    hkv, nb, rows = score.shape
    if hkv != plan.num_kv_heads or rows != plan.num_token_rows:
        raise ValueError(f"score must be [{plan.num_kv_heads}, blocks, {plan.num_token_rows}]")
    if topk_out is not None and (
            topk_out.dtype != torch.int32 or not topk_out.is_contiguous()
            or tuple(topk_out.shape) != (rows, hkv, plan.topk_blocks)
            or topk_out.device != q.device):
        raise ValueError(f"topk_out must be contiguous int32 [{rows}, {hkv}, "
                         f"{plan.topk_blocks}] on q's device")
    head = _run_args(plan, q, kv_cache, block_table, seq_lens, None, out, selects=True)
    _check(load_library().msa_sparse_decode_select_run(
        *head, float(q_scale), float(k_scale), float(v_scale), block_table.data_ptr(),
        seq_lens.data_ptr(), score.data_ptr(), _I64x3(*score.stride()), nb, _ptr(topk_out),
        out.data_ptr(), float(sm_scale), _stream_handle(stream, q.device)))


class _ShapeArgs:
    """The plan attributes the run-argument checks read, for the call that
    takes a static shape instead of a plan."""

    prefill = False

    def __init__(self, shape: "_Shape"):
        self.batch = shape.batch
        self.num_token_rows = shape.num_token_rows or shape.batch * shape.decode_query_len
        self.num_q_heads = shape.num_q_heads
        self.num_kv_heads = shape.num_kv_heads
        self.page_table_stride = shape.page_table_stride
        self.topk_blocks = shape.topk_blocks
        self.dense = shape.topk_blocks == 0
        self.kv_dtype = shape.kv_dtype
        self.q_dtype = shape.q_dtype
        self.handle = None


def msa_sparse_decode_run_noalloc(q: torch.Tensor, kv_cache: torch.Tensor,
                                  block_table: torch.Tensor, seq_lens: torch.Tensor,
                                  topk: Optional[torch.Tensor], out: torch.Tensor, *,
                                  decode_query_len: int, num_q_heads: int, num_kv_heads: int,
                                  topk_blocks: int, kv_dtype: int, sm_scale: float,
                                  num_token_rows: int = 0, num_splits: int = 0,
                                  q_dtype: int = Q_BF16, tile_rows: int = 0,
                                  k_scale: float = 1.0, v_scale: float = 1.0,
                                  q_scale: float = 1.0, stream=None) -> None:
    """``msa_sparse_decode_run`` without a plan, for callers that cannot
    allocate device memory: the split partials live in the library's static
    per-device scratch (calls that overlap on one GPU race).  The batch is
    ``seq_lens``' length and the device is ``q``'s."""
    shape = _Shape(int(seq_lens.shape[0]), decode_query_len, num_token_rows,
                   int(block_table.stride(0)), num_q_heads, num_kv_heads, PAGE_SIZE, HEAD_DIM,
                   topk_blocks, kv_dtype, num_splits, q_dtype, tile_rows)
    args = _ShapeArgs(shape)
    head = _run_args(args, q, kv_cache, block_table, seq_lens, topk, out)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    _check(load_library().msa_sparse_decode_run_noalloc(
        ctypes.byref(shape), int(dev), *head[1:], float(q_scale), float(k_scale),
        float(v_scale), block_table.data_ptr(), seq_lens.data_ptr(), _ptr(topk),
        _strides3(topk), out.data_ptr(), float(sm_scale), _stream_handle(stream, q.device)))


def msa_sparse_decode_attend(plan: DecodePlan, q: torch.Tensor, kv_cache: torch.Tensor,
                             block_table: torch.Tensor, seq_lens: torch.Tensor,
                             topk: torch.Tensor, out: torch.Tensor, *, sm_scale: float,
                             k_scale: float = 1.0, v_scale: float = 1.0,
                             q_scale: float = 1.0, stream=None) -> None:
    """First launch of a step (see ``msa_sparse_decode_run``)."""
    _require_decode_plan(plan)
    head = _run_args(plan, q, kv_cache, block_table, seq_lens, topk, out)
    _check(load_library().msa_sparse_decode_attend(
        *head, float(q_scale), float(k_scale), float(v_scale), block_table.data_ptr(), seq_lens.data_ptr(),
        _ptr(topk), _strides3(topk), out.data_ptr(), float(sm_scale),
        _stream_handle(stream, q.device)))


def msa_sparse_decode_merge(plan: DecodePlan, out: torch.Tensor, *, v_scale: float = 1.0,
                            stream=None) -> None:
    """Second launch of a step: merge the split partials into ``out``."""
    _check_q(out, "out", plan.num_token_rows, plan.num_q_heads)
    _check(load_library().msa_sparse_decode_merge(plan.handle, out.data_ptr(), float(v_scale),
                                                  _stream_handle(stream, out.device)))


def msa_block_score_topk(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, *, decode_query_len: int, num_kv_heads: int,
                         max_blocks: int, score: torch.Tensor,
                         topk_out: Optional[torch.Tensor], k_scale: float = 1.0,
                         q_scale: float = 1.0, num_token_rows: int = 0,
                         kv_dtype: Optional[int] = None, stream=None) -> None:
    """score[h, b, t] (logical; any strides) and topk_out[t, h, :] for every row
    (topk_out=None: the scores alone, for msa_sparse_decode_select_run).
    The q format follows q's dtype; a uint8 cache is e4m3 unless ``kv_dtype``
    says otherwise."""
    batch = int(seq_lens.shape[0])
    rows = num_token_rows or batch * decode_query_len
    q_dtype = _q_dtype_of(q)
    _check_q(q, "q", rows, q.shape[1] if q.dim() == 3 else -1, q_dtype)
    kvd = _kv_dtype_of(kv_cache, kv_dtype)
    _check_kv(kv_cache, num_kv_heads, kvd)
    _check_tables(block_table, seq_lens, batch)
    if score.dtype != torch.float32 or score.dim() != 3 or \
            tuple(score.shape) != (num_kv_heads, max_blocks, rows):
        raise ValueError(f"score must be float32 [{num_kv_heads}, {max_blocks}, {rows}]")
    if topk_out is not None and (
            topk_out.dtype != torch.int32 or not topk_out.is_contiguous()
            or topk_out.dim() != 3 or topk_out.shape[0] != rows
            or topk_out.shape[1] != num_kv_heads):
        raise ValueError(f"topk_out must be contiguous int32 [{rows}, {num_kv_heads}, k]")
    k = int(topk_out.shape[2]) if topk_out is not None else 0
    shape = _Shape(batch, decode_query_len, rows, block_table.stride(0), q.shape[1],
                   num_kv_heads, PAGE_SIZE, HEAD_DIM, k, kvd, 0, q_dtype)
    _check(load_library().msa_block_score_topk(
        ctypes.byref(shape), q.data_ptr(), kv_cache.data_ptr(), _kv_strides(kv_cache, kvd),
        kv_cache.shape[0], float(q_scale), float(k_scale), block_table.data_ptr(), seq_lens.data_ptr(),
        int(max_blocks), score.data_ptr(), _I64x3(*score.stride()), _ptr(topk_out), k,
        _stream_handle(stream, q.device)))


def msa_topk_select(score: torch.Tensor, topk_out: torch.Tensor, stream=None) -> None:
    """topk_out[t, h, :] from a float32 logical [Hkv, max_blocks, rows] score."""
    if score.dtype != torch.float32 or score.dim() != 3 or score.device.type != "cuda":
        raise ValueError("score must be a 3-D float32 device tensor [Hkv, blocks, rows]")
    hkv, nb, rows = score.shape
    if topk_out.dtype != torch.int32 or not topk_out.is_contiguous() or \
            tuple(topk_out.shape[:2]) != (rows, hkv):
        raise ValueError(f"topk_out must be contiguous int32 [{rows}, {hkv}, k]")
    _check(load_library().msa_topk_select(
        score.data_ptr(), _I64x3(*score.stride()), hkv, nb, rows, topk_out.data_ptr(),
        int(topk_out.shape[2]), _stream_handle(stream, score.device)))


def _fp8_to_bf16(fn_name, typed, inp: torch.Tensor, out: torch.Tensor, stream) -> None:
    if inp.dtype not in (torch.uint8, typed) or not inp.is_contiguous():
        raise ValueError(f"inp must be contiguous uint8 / {typed}")
    if out.dtype != torch.bfloat16 or not out.is_contiguous() or out.numel() != inp.numel():
        raise ValueError("out must be contiguous bfloat16 with inp's element count")
    _check(getattr(load_library(), fn_name)(inp.data_ptr(), out.data_ptr(), inp.numel(),
                                            _stream_handle(stream, inp.device)))


def msa_fp8_e4m3_to_bf16(inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _fp8_to_bf16("msa_fp8_e4m3_to_bf16", torch.float8_e4m3fn, inp, out, stream)


def msa_fp8_e5m2_to_bf16(inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _fp8_to_bf16("msa_fp8_e5m2_to_bf16", torch.float8_e5m2, inp, out, stream)


def msa_mxfp4_to_bf16(kv_cache: torch.Tensor, out: torch.Tensor, *, num_kv_heads: int,
                      stream=None) -> None:
    """out[p, h, i, :] = packed bf16 K|V row i of head h on page p of a 4-bit
    head-slot cache (block scales applied, global scales not)."""
    _check_kv(kv_cache, num_kv_heads, KV_MXFP4)
    nb = kv_cache.shape[0]
    if (out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != kv_cache.device
            or tuple(out.shape) != (nb, num_kv_heads, PAGE_SIZE, 2 * HEAD_DIM)):
        raise ValueError(f"out must be contiguous bfloat16 ({nb}, {num_kv_heads}, 128, 256) "
                         "on the cache's device")
    _check(load_library().msa_mxfp4_to_bf16(
        kv_cache.data_ptr(), _kv_strides(kv_cache, KV_MXFP4), nb, int(num_kv_heads),
        out.data_ptr(), _stream_handle(stream, kv_cache.device)))


class PlanCache:
    """Plans keyed by (batch, decode_query_len, page_table_stride, num_q_heads,
    num_kv_heads, page_size, topk_blocks) -- the key of
    ``MSACutlassDecodePlanCache.prepare`` -- plus kv and q dtypes, padding rows
    and split count."""

    def __init__(self):
        self.plans = {}

    def prepare(self, block_table: torch.Tensor, seq_lens: torch.Tensor,
                decode_query_len: int, *, num_q_heads: int, num_kv_heads: int,
                topk_blocks: int, kv_dtype: int, page_size: int = PAGE_SIZE,
                num_token_rows: int = 0, num_splits: int = 0,
                q_dtype: int = Q_BF16) -> DecodePlan:
        batch = int(seq_lens.shape[0])
        _check_tables(block_table, seq_lens, batch)
        stride = int(block_table.stride(0))
        key = (batch, decode_query_len, stride, num_q_heads, num_kv_heads, page_size,
               topk_blocks, kv_dtype, num_token_rows, num_splits, q_dtype)
        plan = self.plans.get(key)
        if plan is None:
            plan = msa_sparse_decode_plan(
                batch, decode_query_len, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                page_table_stride=stride, topk_blocks=topk_blocks, kv_dtype=kv_dtype,
                num_token_rows=num_token_rows, num_splits=num_splits, page_size=page_size,
                q_dtype=q_dtype, device=block_table.device)
            self.plans[key] = plan
        return plan


def msa_probe_read_runs(buffer: torch.Tensor, run_offsets: torch.Tensor,
                        run_bytes: torch.Tensor, wg_first_run: torch.Tensor,
                        out: torch.Tensor, stream=None) -> None:
    """Memory-rate probe: workgroup w reads the byte runs
    wg_first_run[w] .. wg_first_run[w+1]-1 of ``buffer`` (offsets int64, sizes
    int32) and writes the XOR of the 32-bit words it read to out[2w] and its
    count of skipped runs to out[2w+1] (out int32 [2 * workgroups])."""
    dev = buffer.device
    if dev.type != "cuda" or not buffer.is_contiguous():
        raise ValueError("buffer must be a contiguous device tensor")
    for name, t, dt in (("run_offsets", run_offsets, torch.int64),
                        ("run_bytes", run_bytes, torch.int32),
                        ("wg_first_run", wg_first_run, torch.int32),
                        ("out", out, torch.int32)):
        if t.dtype != dt or t.dim() != 1 or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous 1-D {dt} tensor on the buffer's "
                             "device")
    if run_offsets.numel() != run_bytes.numel():
        raise ValueError("run_offsets and run_bytes must have the same length")
    wgs = wg_first_run.numel() - 1
    if wgs < 0 or out.numel() != 2 * wgs:
        raise ValueError("wg_first_run needs workgroups + 1 entries and out 2 * workgroups")
    _check(load_library().msa_probe_read_runs(
        buffer.data_ptr(), buffer.numel() * buffer.element_size(), run_offsets.data_ptr(),
        run_bytes.data_ptr(), run_offsets.numel(), wg_first_run.data_ptr(), wgs,
        out.data_ptr(), _stream_handle(stream, dev)))
