"""Helpers shared by the GPU parity tests: move a seeded case to the device,
run the HIP path through the C ABI, and compare with the float64 oracle."""
import numpy as np
import torch

import block_sparse_gqa_decode_amd as msa
from oracle import msa_oracle as om
from workloads import gen

ATOL = 1e-2
RTOL = 1e-2

KV_CODES = {gen.KV_FP8: msa.KV_FP8_E4M3, gen.KV_E5M2: msa.KV_FP8_E5M2, gen.KV_BF16: msa.KV_BF16,
            gen.KV_MXFP4: msa.KV_MXFP4}
Q_CODES = {gen.Q_BF16: msa.Q_BF16, gen.Q_FP8: msa.Q_FP8_E4M3}


class DevCase:
    def __init__(self, case: gen.DecodeCase, dev="cuda:0", layout="hnd"):
        self.case = case
        self.dev = torch.device(dev)
        if case.kv_dtype in (gen.KV_FP8, gen.KV_MXFP4):
            kv = torch.from_numpy(case.kv)                       # uint8 codes / head slots
        elif case.kv_dtype == gen.KV_E5M2:
            kv = torch.from_numpy(case.kv).view(torch.float8_e5m2)
        else:
            kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16)
        if layout == "nhd":
            assert case.kv_dtype != gen.KV_MXFP4, "4-bit pages have one layout"
            # physical (num_blocks, 128, Hkv, 256), viewed logically as HND
            kv = kv.permute(0, 2, 1, 3).contiguous().to(self.dev).permute(0, 2, 1, 3)
        else:
            kv = kv.to(self.dev)
        self.kv = kv
        if case.q_dtype == gen.Q_FP8:
            self.q = torch.from_numpy(case.q).view(torch.float8_e4m3fn).to(self.dev)
        else:
            self.q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(self.dev)
        self.block_table = torch.from_numpy(case.block_table).to(self.dev)
        self.seq_lens = torch.from_numpy(case.seq_lens).to(self.dev)
        self.topk = (torch.from_numpy(case.topk).to(self.dev)
                     if case.topk is not None else None)
        self.out = self.new_out()

    def new_out(self):
        """A bf16 output tensor of q's shape, filled with NaN."""
        return torch.full(tuple(self.q.shape), float("nan"), dtype=torch.bfloat16,
                          device=self.dev)

    @property
    def kv_dtype(self):
        return KV_CODES[self.case.kv_dtype]

    @property
    def q_dtype(self):
        return Q_CODES[self.case.q_dtype]

    def plan(self, num_splits=0, tile_rows=0, dense=False):
        c = self.case
        return msa.msa_sparse_decode_plan(
            c.batch, c.dql, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
            page_table_stride=self.block_table.stride(0), topk_blocks=0 if dense else c.topk_k,
            kv_dtype=self.kv_dtype, num_token_rows=c.num_token_rows, num_splits=num_splits,
            q_dtype=self.q_dtype, tile_rows=tile_rows, device=self.dev)

    def run(self, plan, topk=None, out=None, stream=None):
        c = self.case
        out = self.out if out is None else out
        tk = None if plan.dense else (self.topk if topk is None else topk)
        msa.msa_sparse_decode_run(plan, self.q, self.kv, self.block_table, self.seq_lens,
                                  tk, out,
                                  sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale,
                                  q_scale=c.q_scale, stream=stream)
        return out

    def score(self, score, topk_out, max_blocks, num_token_rows=0, stream=None):
        """Indexer scores + top-k through the C ABI with the case's formats."""
        c = self.case
        msa.msa_block_score_topk(self.q, self.kv, self.block_table, self.seq_lens,
                                 decode_query_len=c.dql, num_kv_heads=c.num_kv_heads,
                                 max_blocks=max_blocks, score=score, topk_out=topk_out,
                                 k_scale=c.k_scale, q_scale=c.q_scale,
                                 num_token_rows=num_token_rows, kv_dtype=self.kv_dtype,
                                 stream=stream)


def oracle_attend(case: gen.DecodeCase, rows=None, topk=None):
    return om.sparse_decode(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                            case.block_table, case.seq_lens,
                            case.topk if topk is None else topk, case.dql,
                            case.num_kv_heads, case.sm_scale, rows=rows,
                            q_dtype=case.q_dtype, q_scale=case.q_scale)


def oracle_dense(case: gen.DecodeCase, rows=None):
    return om.dense_decode(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                           case.block_table, case.seq_lens, case.dql, case.num_kv_heads,
                           case.sm_scale, rows=rows, q_dtype=case.q_dtype,
                           q_scale=case.q_scale)


def oracle_scores(case: gen.DecodeCase, max_blocks, rows=None):
    return om.block_max_scores(case.q, case.kv, case.kv_dtype, case.k_scale, case.block_table,
                               case.seq_lens, case.dql, case.num_kv_heads, max_blocks,
                               rows=rows, q_dtype=case.q_dtype, q_scale=case.q_scale)


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def assert_parity(got: np.ndarray, ref: np.ndarray, atol=ATOL, rtol=RTOL, what=""):
    """max |got-ref| <= atol, ||got-ref|| <= rtol*||ref||, and elementwise
    |got-ref| <= atol + rtol*|ref|."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else 0.0
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} n={diff.size}",
          flush=True)
    assert max_abs <= atol, f"{what}: max abs err {max_abs}"
    assert rel <= rtol, f"{what}: relative L2 err {rel}"
    assert np.all(diff <= atol + rtol * np.abs(ref)), f"{what}: elementwise tolerance"
    return max_abs, rel


class PrefillDevCase:
    """A gen.PrefillCase on the device, run through msa_sparse_prefill_run."""

    def __init__(self, case: gen.PrefillCase, dev="cuda:0"):
        self.case = case
        self.dev = torch.device(dev)
        if case.kv_dtype in (gen.KV_FP8, gen.KV_MXFP4):
            kv = torch.from_numpy(case.kv)
        elif case.kv_dtype == gen.KV_E5M2:
            kv = torch.from_numpy(case.kv).view(torch.float8_e5m2)
        else:
            kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16)
        self.kv = kv.to(self.dev)
        if case.q_dtype == gen.Q_FP8:
            self.q = torch.from_numpy(case.q).view(torch.float8_e4m3fn).to(self.dev)
        else:
            self.q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(self.dev)
        self.block_table = torch.from_numpy(case.block_table).to(self.dev)
        self.cu = torch.from_numpy(case.cu_seqlens_q).to(self.dev)
        self.ctx = torch.from_numpy(case.context_lens).to(self.dev)
        self.topk = torch.from_numpy(case.topk).to(self.dev)
        self.out = torch.full(tuple(self.q.shape), float("nan"), dtype=torch.bfloat16,
                              device=self.dev)

    def plan(self, num_splits=0, tile_rows=0):
        c = self.case
        return msa.msa_sparse_prefill_plan(
            c.batch, c.num_token_rows, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
            page_table_stride=self.block_table.stride(0), topk_blocks=c.topk_k,
            kv_dtype=KV_CODES[c.kv_dtype], q_dtype=Q_CODES[c.q_dtype], num_splits=num_splits,
            tile_rows=tile_rows, device=self.dev)

    def run(self, plan, out=None, stream=None):
        c = self.case
        out = self.out if out is None else out
        msa.msa_sparse_prefill_run(plan, self.q, self.kv, self.block_table, self.cu, self.ctx,
                                   self.topk, out, sm_scale=c.sm_scale, k_scale=c.k_scale,
                                   v_scale=c.v_scale, q_scale=c.q_scale, stream=stream)
        return out


def oracle_prefill(case: gen.PrefillCase, rows=None):
    return om.sparse_prefill(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                             case.block_table, case.cu_seqlens_q, case.context_lens, case.topk,
                             case.num_kv_heads, case.sm_scale, rows=rows, q_dtype=case.q_dtype,
                             q_scale=case.q_scale)
