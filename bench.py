#!/usr/bin/env python3
"""Benchmark of the block-sparse GQA decode attend on one MI355X.

Metric: decode tokens/s and effective KV GB/s (% of HBM peak) of the sparse
GQA attend.  Default workload: the TP4-shaped fp8 decode (batch 32, decode
query length 4, 16 q heads / 1 kv head, head dim 128, page 128, top-16,
fp8 e4m3 packed K|V cache, seq_lens uniform in [16384, 65536]).

A step is one call of ``msa_sparse_decode_run`` (page gather, fp8 dequant,
MFMA QK^T / PV, online softmax, split-K with the fused log-sum-exp merge and
zeroed padding rows: one kernel launch) over one batch.  Timing:

* R independent (q, top-k) replicas, each over its own device copy of the KV
  pool, so a cycle of R steps touches more bytes than the 256 MiB MALL holds
  and pages are read from HBM;
* all R steps are captured in one HIP graph; W warm-up steps, then exactly K
  timed steps between two synchronisations, timed with HIP events recorded on
  the stream the kernels run on (and with the host clock as a cross-check);
* algorithmic bytes per step = every live (token, kv head, selected page)'s
  visible K|V rows + q + out + indices + block-table entries (the bytes the
  attend must move as defined per token), and the unique-page lower bound.

Cross-checks in the same line: one step replayed alone right after a 1 GiB
scrub write (cold) and again straight after (warm), and the float64 oracle
timed on host cores, single-threaded and over a process pool (the pool runs
in a child process started before this one touches the GPU).

With --profile-mode the script instead launches eagerly (no graph) a few
steps for rocprofv3 kernel traces and counters; --copy-calibration runs a
plain device copy of known size for the counter scale factor.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and effective KV GB/s (% HBM peak), sparse GQA attend, 1 GPU"
HBM_PEAK_GBS = 8000.0
# MI355X dense matrix-core peaks (TFLOP/s): index False = bf16, True = fp8.
MFMA_PEAK_TFLOPS = {False: 2500.0, True: 5000.0}
# The headline workload is the largest attend workload (dql 32, ragged,
# 516 token rows); every other workload is reported beside it.
DEFAULT_CONFIG = "c4_spec_ragged"
OTHER_CONFIGS = ("c2_tp4_fp8", "c3_tp1_fp8", "c2_tp4_fp8q", "c2_tp4_e5m2",
                 "c2_tp4_mxfp4", "c2_tp4_mxfp4_fp8q", "pf1_chunked_prefill", "d1_dense_tp1")
FULL_STEP_CONFIG = "c5_full_step"
# Fewest steps ever timed, whatever --steps asks (the timed window then spans
# at least this many step replays).
MIN_TIMED_STEPS = 200
# Shortest timed window.  After the host has left the GPU idle for a second
# or two (generating a workload), the first ~30 ms of replays run up to 10%
# slower than the steady state (c4: 90 us per step over the first 160 steps,
# 80.7 us from about the 400th on), so a window of a few ms measures mostly
# that ramp.  The window is therefore stretched, in whole replays, to at least
# this long, estimated from the warmup replays' own duration.
MIN_TIMED_MS = 300.0


def timed_window(g, steps: int, warmup: int, replicas: int) -> int:
    """Run the warmup replays of graph g (each replays all `replicas` steps)
    and return how many replays to time: --steps rounded up to at least
    MIN_TIMED_STEPS steps and to MIN_TIMED_MS of replays at the warmup's
    rate, in whole replays."""
    import torch

    warm = max(1, (warmup + replicas - 1) // replicas)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(warm):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return window_replays(ev0.elapsed_time(ev1) / warm, steps, replicas)


def window_replays(per_replay_ms: float, steps: int, replicas: int) -> int:
    """Replays to time: enough for --steps (at least MIN_TIMED_STEPS) and for
    MIN_TIMED_MS at per_replay_ms a replay, in whole replays."""
    by_steps = (max(steps, MIN_TIMED_STEPS) + replicas - 1) // replicas
    by_time = int(math.ceil(MIN_TIMED_MS / max(per_replay_ms, 1e-3)))
    return max(1, by_steps, min(by_time, 200000))
# rocprofv3 counter summaries (HBM bytes per launch), one file per workload,
# each valid only for the kernel sources it was taken on.
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "attend": ("block_sparse_gqa_decode_amd/csrc/msa_attend.hip",
               "block_sparse_gqa_decode_amd/csrc/msa_page.h",
               "block_sparse_gqa_decode_amd/csrc/msa_rows.h",
               "block_sparse_gqa_decode_amd/csrc/msa_select.h",
               "block_sparse_gqa_decode_amd/csrc/msa_device.h",
               "block_sparse_gqa_decode_amd/csrc/msa_internal.h"),
    "score": ("block_sparse_gqa_decode_amd/csrc/msa_score.hip",
              "block_sparse_gqa_decode_amd/csrc/msa_page.h",
              "block_sparse_gqa_decode_amd/csrc/msa_select.h",
              "block_sparse_gqa_decode_amd/csrc/msa_device.h",
              "block_sparse_gqa_decode_amd/csrc/msa_internal.h"),
    # the multi-row tile kernel (c4, pf1, d1 plans)
    "tile": ("block_sparse_gqa_decode_amd/csrc/msa_tile.hip",
             "block_sparse_gqa_decode_amd/csrc/msa_page.h",
             "block_sparse_gqa_decode_amd/csrc/msa_rows.h",
             "block_sparse_gqa_decode_amd/csrc/msa_device.h",
             "block_sparse_gqa_decode_amd/csrc/msa_internal.h"),
}

CONFIG_TEXT = {
    "c1_tiny_bf16": "tiny bf16 decode: B=2, dql=1, 16/1 heads, top-4, seq {512,1000}",
    "c2_tp4_fp8": "TP4-shaped fp8 decode: B=32, dql=4, 16/1 heads, top-16, "
                  "seq U[16384,65536]",
    "c3_tp1_fp8": "TP1-shaped fp8 decode: B=16, dql=4, 64/4 heads, top-16, "
                  "seq U[32768,131072], Zipf-recent indices",
    "c4_spec_ragged": "speculative/ragged fp8 decode: B=16, dql=32, 64/4 heads, top-16, "
                      "8 requests at 131072 + 8 in [200,1900], 4 padding rows",
    "c5_full_step": "full decode step with indexer: B=64, dql=1, 64/4 heads, fp8, seq "
                    "log-normal in [8192,262144]; block-max scores -> top-16 -> attend",
    "c2_tp4_fp8q": "c2 with an fp8 e4m3 query (q_scale 0.5) over the fp8 e4m3 cache: "
                   "fp8 x fp8 MFMA for QK^T",
    "c2_tp4_e5m2": "c2 with a bf16 query over an fp8 e5m2 cache",
    "c2_tp4_mxfp4": "c2 with a bf16 query over a 4-bit MXFP4 head-slot cache (e2m1 + E8M0 "
                    "per 32 dims; k_scale 0.5, v_scale 2.0)",
    "c2_tp4_mxfp4_fp8q": "c2 with an fp8 e4m3 query (q_scale 0.5) over the 4-bit MXFP4 "
                         "cache: fp4 x fp8 scaled MFMA for QK^T",
    "pf1_chunked_prefill": "chunked prefill: 4 requests x 1024-token chunks after a cached "
                           "context of U[16384,65536], 64/4 heads, fp8, top-16 per (token, "
                           "kv head), recent-biased",
    "d1_dense_tp1": "dense decode (every visible block): B=16, dql=4, 64/4 heads, fp8, "
                    "seq U[32768,131072]",
}


def kernel_source_hash(kernel: str = "attend") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# byte accounting
# ---------------------------------------------------------------------------

def kv_half_row_bytes(kv_dtype: str) -> int:
    """Bytes of one key's K (or V) entry: 128 elements, plus the four E8M0
    block scales of a 4-bit row."""
    return {"bf16": 256, "fp8_e4m3": 128, "fp8_e5m2": 128, "mxfp4": 64 + 4}[kv_dtype]


def step_bytes(case, q, topk):
    """Algorithmic bytes of one attend step (see module docstring)."""
    import numpy as np

    row_bytes = 2 * kv_half_row_bytes(case.kv_dtype)
    real = case.real_rows
    t = np.arange(real)
    if hasattr(case, "cu_seqlens_q"):       # ragged prefill rows
        r = np.repeat(np.arange(case.batch), case.q_lens)
        pos = case.positions()
    else:
        r = t // case.dql
        pos = case.seq_lens[r].astype(np.int64) - case.dql + (t % case.dql)
    if topk is None:   # dense: every visible block of every (row, kv head)
        nb_all = int(pos.max()) // 128 + 1 if real else 0
        b = np.broadcast_to(np.arange(nb_all, dtype=np.int64)[None, None, :],
                            (real, case.num_kv_heads, nb_all))
    else:
        b = topk[:real].astype(np.int64)                   # [T, Hkv, k]
    start = b * 128
    live = (b >= 0) & (start <= pos[:, None, None]) & (b < case.block_table.shape[1])
    nvis = np.where(live, np.minimum(128, pos[:, None, None] - start + 1), 0)
    eff_kv = int(nvis.sum()) * row_bytes
    # unique (request, head, block) pages, at their largest visible count
    hh = np.broadcast_to(np.arange(case.num_kv_heads)[None, :, None], b.shape)
    rr = np.broadcast_to(r[:, None, None], b.shape)
    key = (rr[live].astype(np.int64) * case.num_kv_heads + hh[live]) * (1 << 22) + b[live]
    order = np.lexsort((-nvis[live], key))
    ks, nv = key[order], nvis[live][order]
    first = np.ones(len(ks), dtype=bool)
    first[1:] = ks[1:] != ks[:-1]
    uniq_kv = int(nv[first].sum()) * row_bytes
    n_live = int(live.sum())
    key_units = int(nvis.sum())           # (visible key, token row, kv head) triples
    group = case.num_q_heads // case.num_kv_heads
    q_bytes = real * case.num_q_heads * 128 * (1 if case.q_dtype == "fp8_e4m3" else 2)
    out_bytes = case.num_token_rows * case.num_q_heads * 128 * 2
    idx_bytes = 0 if topk is None else real * case.num_kv_heads * case.topk_k * 4
    meta = idx_bytes + n_live * 4 + case.batch * 4
    return {
        "effective_kv": eff_kv,
        "unique_kv": uniq_kv,
        "q_out_meta": q_bytes + out_bytes + meta,
        "algorithmic": eff_kv + q_bytes + out_bytes + meta,
        "unique_algorithmic": uniq_kv + q_bytes + out_bytes + meta,
        "live_pages": n_live,
        # S = q K^T and O += P V: 2 * 128 flops each per (q head, visible key)
        "flops": key_units * 4 * group * 128,
    }


# ---------------------------------------------------------------------------
# device setup
# ---------------------------------------------------------------------------

def _host_kv(case):
    """The case's KV pool as a CPU tensor of the cache's dtype."""
    import numpy as np
    import torch

    if case.kv_dtype in ("fp8_e4m3", "mxfp4"):
        return torch.from_numpy(case.kv)
    if case.kv_dtype == "fp8_e5m2":
        return torch.from_numpy(case.kv).view(torch.float8_e5m2)
    return torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16)


def _host_q(case, qh):
    import numpy as np
    import torch

    if case.q_dtype == "fp8_e4m3":
        return torch.from_numpy(qh).view(torch.float8_e4m3fn)
    return torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16)


def _kv_code(case):
    import block_sparse_gqa_decode_amd as msa

    return {"fp8_e4m3": msa.KV_FP8_E4M3, "fp8_e5m2": msa.KV_FP8_E5M2,
            "bf16": msa.KV_BF16, "mxfp4": msa.KV_MXFP4}[case.kv_dtype]


def _q_code(case):
    import block_sparse_gqa_decode_amd as msa

    return msa.Q_FP8_E4M3 if case.q_dtype == "fp8_e4m3" else msa.Q_BF16


class DeviceSet:
    """R replicas of one step's inputs, each over its own copy of the pool."""

    def __init__(self, case, replicas: int, splits: int, dev, tile_rows: int = 0):
        import numpy as np
        import torch

        import block_sparse_gqa_decode_amd as msa

        self.case = case
        self.prefill = hasattr(case, "cu_seqlens_q")
        self.dense = case.topk is None
        host = _host_kv(case)
        nb = int(case.kv.shape[0])
        self.kv = torch.empty((replicas * nb,) + tuple(host.shape[1:]), dtype=host.dtype,
                              device=dev)
        self.kv[:nb].copy_(host)
        for i in range(1, replicas):
            self.kv[i * nb:(i + 1) * nb].copy_(self.kv[:nb])
        self.seq_lens = torch.from_numpy(case.seq_lens).to(dev)
        if self.prefill:
            self.cu = torch.from_numpy(case.cu_seqlens_q).to(dev)
            self.ctx = torch.from_numpy(case.context_lens).to(dev)
        sets = [(case.q, case.topk)] + list(case.replicas)
        assert len(sets) >= replicas, "not enough replicas generated"
        self.steps = []
        self.bytes = []
        for i in range(replicas):
            qh, tk = sets[i]
            bt = torch.from_numpy((case.block_table.astype(np.int64) + i * nb).astype(
                np.int32)).to(dev)
            q = _host_q(case, qh).to(dev)
            topk = None if tk is None else torch.from_numpy(tk).to(dev)
            out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
            self.steps.append((q, bt, topk, out))
            self.bytes.append(step_bytes(case, qh, tk))
        if self.prefill:
            self.plan = msa.msa_sparse_prefill_plan(
                case.batch, case.num_token_rows, num_q_heads=case.num_q_heads,
                num_kv_heads=case.num_kv_heads, page_table_stride=case.block_table.shape[1],
                topk_blocks=case.topk_k, kv_dtype=_kv_code(case), q_dtype=_q_code(case),
                num_splits=splits, tile_rows=tile_rows, device=dev)
        else:
            self.plan = msa.msa_sparse_decode_plan(
                case.batch, case.dql, num_q_heads=case.num_q_heads,
                num_kv_heads=case.num_kv_heads, page_table_stride=case.block_table.shape[1],
                topk_blocks=0 if self.dense else case.topk_k, kv_dtype=_kv_code(case),
                q_dtype=_q_code(case), num_token_rows=case.num_token_rows, num_splits=splits,
                tile_rows=tile_rows, device=dev)
        self.msa = msa

    def run_step(self, i):
        q, bt, topk, out = self.steps[i]
        c = self.case
        if self.prefill:
            self.msa.msa_sparse_prefill_run(self.plan, q, self.kv, bt, self.cu, self.ctx, topk,
                                            out, sm_scale=c.sm_scale, k_scale=c.k_scale,
                                            v_scale=c.v_scale, q_scale=c.q_scale)
            return
        self.msa.msa_sparse_decode_run(self.plan, q, self.kv, bt, self.seq_lens, topk, out,
                                       sm_scale=c.sm_scale, k_scale=c.k_scale,
                                       v_scale=c.v_scale, q_scale=c.q_scale)

    def run_attend(self, i):
        if self.prefill:   # one launch unless split; the step is the attend
            self.run_step(i)
            return
        q, bt, topk, out = self.steps[i]
        c = self.case
        self.msa.msa_sparse_decode_attend(self.plan, q, self.kv, bt, self.seq_lens, topk, out,
                                          sm_scale=c.sm_scale, k_scale=c.k_scale,
                                          v_scale=c.v_scale, q_scale=c.q_scale)

    def mean_bytes(self, key):
        return sum(b[key] for b in self.bytes) / len(self.bytes)


def cold_and_warm(ds, n: int = 5):
    """One step (replica 0, captured alone) timed right after a 1 GiB scrub
    write (cold: pages come from HBM) and again straight after (warm: pages
    in L2 / MALL); medians over n trials, in ms.  Cross-checks of the rotated
    graph timing, not the reported value."""
    import statistics

    import torch

    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        ds.run_step(0)
    torch.cuda.synchronize()
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=ds.kv.device)
    cold, warm = [], []
    for i in range(n):
        scrub.fill_(float(i))
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        g1.replay()
        e[1].record()
        g1.replay()
        e[2].record()
        torch.cuda.synchronize()
        cold.append(e[0].elapsed_time(e[1]))
        warm.append(e[1].elapsed_time(e[2]))
    del scrub, g1
    return statistics.median(cold), statistics.median(warm)


def make_case(name, extra_replicas):
    """The named workload with extra (q, top-k) replicas."""
    from workloads import gen

    if name in gen.PREFILL_CONFIG_NAMES:
        return gen.make_prefill_config(name, replicas=extra_replicas)
    if name in gen.DENSE_CONFIG_NAMES:
        return gen.make_dense_config(name, replicas=extra_replicas)
    return gen.make_config(name, replicas=extra_replicas)


def time_config(name, steps, warmup, replicas, splits, dev, verbose=True, tile_rows=0,
                cold=False, ceiling=False):
    import torch

    from workloads import gen

    t0 = time.time()
    case = make_case(name, replicas - 1)
    ds = DeviceSet(case, replicas, splits, dev, tile_rows=tile_rows)
    if verbose:
        print(f"[bench] {name}: generated + uploaded in {time.time() - t0:.1f}s "
              f"(pool {case.kv.nbytes / 2**20:.0f} MiB x {replicas}, splits "
              f"{ds.plan.num_splits})", file=sys.stderr, flush=True)

    # Warm the plan on a side stream, then capture the R steps in one graph,
    # and the R attend launches alone in a second graph.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(replicas):
            ds.run_step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(replicas):
            ds.run_step(i)
    attend_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(attend_graph):
        for i in range(replicas):
            ds.run_attend(i)
    torch.cuda.synchronize()

    def timed(g, n_replays):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        ev0.record()
        for _ in range(n_replays):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1), time.perf_counter() - h0

    replays = timed_window(graph, steps, warmup, replicas)
    n_steps = replays * replicas
    gpu_ms, host_s = timed(graph, replays)
    ms_step = gpu_ms / n_steps
    # The attend kernel alone: same launches, without the merge pass (which
    # a single-row plan with 2..4 splits does inside the attend).
    a_replays = timed_window(attend_graph, steps, warmup, replicas)
    attend_ms, _ = timed(attend_graph, a_replays)
    attend_ms /= a_replays * replicas
    eff = ds.mean_bytes("effective_kv")
    uniq = ds.mean_bytes("unique_kv")
    alg = ds.mean_bytes("algorithmic")
    s = ms_step / 1e3
    res = {
        "config": name,
        "steps": n_steps,
        "steps_requested": steps,
        "ms_per_step": ms_step,
        "host_ms_per_step": host_s * 1e3 / n_steps,
        "tokens_per_s": case.real_rows / s,
        "effective_kv_gbs": eff / s / 1e9,
        "unique_kv_gbs": uniq / s / 1e9,
        "algorithmic_gbs": alg / s / 1e9,
        "effective_kv_bytes": eff,
        "unique_kv_bytes": uniq,
        "algorithmic_bytes": alg,
        "unique_algorithmic_bytes": ds.mean_bytes("unique_algorithmic"),
        "attend_flops": ds.mean_bytes("flops"),
        "splits": ds.plan.num_splits,
        "tile_rows": ds.plan.tile_rows,
        "launches_per_step": 1 if ds.plan.num_splits == 1 or ds.plan.merges_in_attend else 2,
        "attend_ms": attend_ms,
        "real_rows": case.real_rows,
    }
    res["unique_pct_peak"] = 100.0 * res["unique_kv_gbs"] / HBM_PEAK_GBS
    del graph, attend_graph
    if ceiling and not ds.prefill and not ds.dense and ds.plan.tile_rows == 1 \
            and case.kv_dtype != "mxfp4":
        res["measured_ceiling"] = gather_ceiling(ds, replicas, steps, warmup, attend_ms)
    if cold:
        res["cold_ms_per_step"], res["warm_ms_per_step"] = cold_and_warm(ds)
    return res, case


def _xcd_chunk(units: int, hkv: int) -> int:
    c = units // 8 if units // 8 < hkv * 16 else hkv * 16
    return c if c > 1 else 1


def attend_page_runs(ds, replica: int):
    """The byte runs the single-row attend reads for one replica, per
    workgroup id of its launch: the visible K|V rows of each live page of the
    workgroup's (unit, split) share, in the order it streams them.  Mirrors
    the launch's deal of units to XCD slots (chunks of consecutive units, all
    splits of a unit in one slot) and the split of a unit's live list into
    equal consecutive shares."""
    import numpy as np

    case = ds.case
    kv = ds.kv
    es = kv.element_size()
    s0, s1, s2 = (kv.stride(i) * es for i in range(3))
    row_bytes = 2 * kv_half_row_bytes(case.kv_dtype)
    assert s2 == row_bytes, "rows of a page-head must be contiguous"
    nb_total = kv.shape[0]
    _, bt, _, _ = ds.steps[replica]
    bt = bt.cpu().numpy()
    topk = ([case.topk] + [tk for _, tk in case.replicas])[replica]
    hkv, k, dql = case.num_kv_heads, case.topk_k, case.dql
    units = case.num_token_rows * hkv
    S = ds.plan.num_splits
    c = _xcd_chunk(units, hkv)
    groups = (units + 8 * c - 1) // (8 * c) * c
    grid = groups * 8 * S
    offs, lens, first = [], [], [0]
    for wg in range(grid):
        xslot, q8 = wg % 8, wg // 8
        split, kk = q8 % S, q8 // S
        unit = ((kk // c) * 8 + xslot) * c + kk % c
        if unit < units and unit // hkv < case.real_rows:
            t, h = divmod(unit, hkv)
            r = t // dql
            pos = int(case.seq_lens[r]) - dql + t % dql
            live = []
            for b in topk[t, h, :k]:
                b = int(b)
                if 0 <= b < bt.shape[1] and b * 128 <= pos:
                    pg = int(bt[r, b])
                    if 0 <= pg < nb_total:
                        live.append((pg, min(128, pos - b * 128 + 1)))
            per = (len(live) + S - 1) // S
            lo = min(len(live), split * per)
            for pg, nvis in live[lo:min(len(live), lo + per)]:
                base, n = pg * s0 + h * s1, nvis * row_bytes
                for o in range(0, n, 32768):
                    offs.append(base + o)
                    lens.append(min(32768, n - o))
        first.append(len(offs))
    return (np.array(offs, dtype=np.int64), np.array(lens, dtype=np.int32),
            np.array(first, dtype=np.int32))


def contiguous_runs(lens, first, base: int, span: int):
    """Runs of the same per-workgroup byte counts laid end to end from base
    (wrapping inside [base, base + span)), cut at 32 KiB: a plain streaming
    read."""
    import numpy as np

    offs, clens, cfirst = [], [], [0]
    cur = 0
    for w in range(len(first) - 1):
        n = int(lens[first[w]:first[w + 1]].astype(np.int64).sum())
        for o in range(0, n, 32768):
            if cur + 32768 > span:
                cur = 0
            offs.append(base + cur)
            clens.append(min(32768, n - o))
            cur += clens[-1]
        cfirst.append(len(offs))
    return (np.array(offs, dtype=np.int64), np.array(clens, dtype=np.int32),
            np.array(cfirst, dtype=np.int32))


def gather_ceiling(ds, replicas: int, steps: int, warmup: int, attend_ms: float):
    """Time the memory-rate probe over exactly the attend's K|V rows (same
    workgroup ids, pages and order; no top-k or block-table lookups, no
    compute, no merge), then over contiguous runs of the same sizes.  The
    probe's checksums for replica 0 are checked against numpy first."""
    import numpy as np
    import torch

    import block_sparse_gqa_decode_amd as msa

    dev = ds.kv.device
    kvb = ds.kv.view(torch.uint8) if ds.kv.dtype != torch.uint8 else ds.kv
    kvb = kvb.reshape(-1)
    pool_bytes = kvb.numel() // replicas
    sets = {"gather": [], "contiguous": []}
    kv_bytes = []
    for i in range(replicas):
        offs, lens, first = attend_page_runs(ds, i)
        kv_bytes.append(float(lens.astype(np.int64).sum()))
        sets["gather"].append((offs, lens, first))
        sets["contiguous"].append(contiguous_runs(lens, first, i * pool_bytes, pool_bytes))
    host0 = None
    res = {"kv_bytes_per_step": sum(kv_bytes) / replicas}
    for kind, lists in sets.items():
        dev_sets = []
        for offs, lens, first in lists:
            out = torch.zeros(2 * (len(first) - 1), dtype=torch.int32, device=dev)
            dev_sets.append((torch.from_numpy(offs).to(dev), torch.from_numpy(lens).to(dev),
                             torch.from_numpy(first).to(dev), out))

        def launch(i):
            o, ln, f, out = dev_sets[i]
            msa.msa_probe_read_runs(kvb, o, ln, f, out)

        for i in range(replicas):
            launch(i)
        torch.cuda.synchronize()
        if kind == "gather":
            # bit-exact check of what replica 0's probe read
            if host0 is None:
                host0 = kvb[:pool_bytes].cpu().numpy()
            offs, lens, first = lists[0]
            words = host0.view(np.uint32)
            got = dev_sets[0][3].cpu().numpy().view(np.uint32)
            for w in range(len(first) - 1):
                x = np.uint32(0)
                for j in range(first[w], first[w + 1]):
                    x ^= np.bitwise_xor.reduce(words[offs[j] // 4:(offs[j] + lens[j]) // 4])
                assert got[2 * w] == x and got[2 * w + 1] == 0, "probe read other bytes"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(replicas):
                launch(i)
        reps = timed_window(g, steps, warmup, replicas)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * replicas)
        res[f"{kind}_us"] = round(us, 3)
        res[f"{kind}_gbs"] = round(res["kv_bytes_per_step"] / us / 1e3, 1)
        del g
    res["attend_us"] = round(attend_ms * 1e3, 3)
    res["gather_share_of_attend"] = round(res["gather_us"] / res["attend_us"], 4)
    res["note"] = ("msa_probe_read_runs, graph replays over the same replicas: 'gather' "
                   "reads exactly the attend's live K|V rows with the attend's workgroup "
                   "ids and page order and nothing else; 'contiguous' reads the same "
                   "per-workgroup byte counts as a plain streaming read. Checksums of "
                   "replica 0 verified against numpy.")
    return res


def scorer_bytes(case):
    """Algorithmic bytes of the indexer step: the K half of every visible page
    of every (request, kv head), q, the score write and its read by the
    selector, and the top-k write."""
    import numpy as np

    kv_rows = 0
    for r in range(case.batch):
        pos_last = int(case.seq_lens[r]) - 1
        nb = pos_last // 128 + 1
        kv_rows += (nb - 1) * 128 + (pos_last - (nb - 1) * 128 + 1)
    k_bytes = kv_rows * case.num_kv_heads * kv_half_row_bytes(case.kv_dtype)
    q_bytes = case.real_rows * case.num_q_heads * 128 * (1 if case.q_dtype == "fp8_e4m3" else 2)
    score_bytes = case.num_kv_heads * case.max_blocks * case.num_token_rows * 4
    topk_bytes = case.num_token_rows * case.num_kv_heads * case.topk_k * 4
    table_bytes = int(np.sum((case.seq_lens.astype(np.int64) + 127) // 128)) * 4 * \
        case.num_kv_heads
    scorer = k_bytes + q_bytes + score_bytes + table_bytes
    selector = score_bytes + topk_bytes
    # Matrix-core work: one 16-row S^T tile (the group's q heads, padded to
    # the MFMA's 16 rows) against all 128 keys of every scored block.
    items = int(np.sum((case.seq_lens.astype(np.int64) + 127) // 128)) * \
        case.num_kv_heads * case.dql
    mfma_flops = items * 2 * 16 * 128 * 128
    return {"k_half": k_bytes, "scorer": scorer, "selector": selector,
            "score_read": score_bytes, "topk": topk_bytes, "algorithmic": scorer + selector,
            "mfma_flops": mfma_flops}


class FullStepSet:
    """R replicas of the full decode step with the indexer: block-max scores ->
    top-k -> attend, each replica over its own copy of the pool."""

    def __init__(self, case, replicas: int, dev):
        import numpy as np
        import torch

        import block_sparse_gqa_decode_amd as msa

        self.case, self.msa = case, msa
        host = _host_kv(case)
        nb = case.num_blocks
        self.kv = torch.empty((replicas * nb,) + tuple(host.shape[1:]), dtype=host.dtype,
                              device=dev)
        self.kv[:nb].copy_(host)
        for i in range(1, replicas):
            self.kv[i * nb:(i + 1) * nb].copy_(self.kv[:nb])
        self.seq_lens = torch.from_numpy(case.seq_lens).to(dev)
        qs = [case.q] + [qh for qh, _ in case.replicas]
        rows = case.num_token_rows
        self.sets = []
        for i in range(replicas):
            bt = torch.from_numpy((case.block_table.astype(np.int64) + i * nb).astype(
                np.int32)).to(dev)
            q = _host_q(case, qs[i]).to(dev)
            # physical [Hkv, rows, blocks] so that the selector's row reads are
            # contiguous; passed as the logical [Hkv, blocks, rows] view
            score = torch.empty((case.num_kv_heads, rows, case.max_blocks), dtype=torch.float32,
                                device=dev).transpose(1, 2)
            sel = torch.empty((rows, case.num_kv_heads, case.topk_k), dtype=torch.int32,
                              device=dev)
            self.sets.append((q, bt, score, sel, torch.empty(tuple(q.shape),
                                                             dtype=torch.bfloat16, device=dev)))
        self.plan = msa.msa_sparse_decode_plan(
            case.batch, case.dql, num_q_heads=case.num_q_heads,
            num_kv_heads=case.num_kv_heads, page_table_stride=case.block_table.shape[1],
            topk_blocks=case.topk_k, kv_dtype=_kv_code(case), q_dtype=_q_code(case),
            device=dev)

    def run_score(self, i):
        q, bt, score, sel, _ = self.sets[i]
        c = self.case
        self.msa.msa_block_score_topk(q, self.kv, bt, self.seq_lens, decode_query_len=c.dql,
                                      num_kv_heads=c.num_kv_heads, max_blocks=c.max_blocks,
                                      score=score, topk_out=sel, k_scale=c.k_scale,
                                      q_scale=c.q_scale, kv_dtype=_kv_code(case=c))

    def run_attend(self, i):
        q, bt, _, sel, out = self.sets[i]
        c = self.case
        self.msa.msa_sparse_decode_run(self.plan, q, self.kv, bt, self.seq_lens, sel, out,
                                       sm_scale=c.sm_scale, k_scale=c.k_scale,
                                       v_scale=c.v_scale, q_scale=c.q_scale)

    def run_select(self, i):
        _, _, score, sel, _ = self.sets[i]
        self.msa.msa_topk_select(score, sel)

    def run_score_only(self, i):
        q, bt, score, _, _ = self.sets[i]
        c = self.case
        self.msa.msa_block_score_topk(q, self.kv, bt, self.seq_lens, decode_query_len=c.dql,
                                      num_kv_heads=c.num_kv_heads, max_blocks=c.max_blocks,
                                      score=score, topk_out=None, k_scale=c.k_scale,
                                      q_scale=c.q_scale, kv_dtype=_kv_code(case=c))

    def run_select_attend(self, i):
        q, bt, score, _, out = self.sets[i]
        c = self.case
        self.msa.msa_sparse_decode_select_run(self.plan, q, self.kv, bt, self.seq_lens, score,
                                              out, sm_scale=c.sm_scale, k_scale=c.k_scale,
                                              v_scale=c.v_scale, q_scale=c.q_scale)

    def run_step_separate(self, i):
        """Three launches: scores, the selector, the attend over its top-k."""
        self.run_score(i)
        self.run_attend(i)

    def run_step(self, i):
        """Two launches: scores, then the attend that selects its own top-k."""
        self.run_score_only(i)
        self.run_select_attend(i)


def _graph_time(fns, replicas, steps, warmup):
    """HIP-event time per step of graph replays of fns over the R replicas."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(replicas):
            fns(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(replicas):
            fns(i)
    torch.cuda.synchronize()
    replays = timed_window(g, steps, warmup, replicas)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(replays):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / (replays * replicas)
    del g
    return ms, replays * replicas


def time_full_step(name, steps, warmup, replicas, dev, verbose=True):
    """The full decode step with the indexer (score -> top-k -> attend)."""
    import torch

    from workloads import gen

    t0 = time.time()
    case = gen.make_config(name, replicas=replicas - 1)
    fs = FullStepSet(case, replicas, dev)
    if verbose:
        print(f"[bench] {name}: generated + uploaded in {time.time() - t0:.1f}s "
              f"(pool {case.kv.nbytes / 2**20:.0f} MiB x {replicas}, max_blocks "
              f"{case.max_blocks})", file=sys.stderr, flush=True)
    step_ms, n = _graph_time(fs.run_step, replicas, steps, warmup)
    separate_ms, _ = _graph_time(fs.run_step_separate, replicas, steps, warmup)
    score_ms, _ = _graph_time(fs.run_score, replicas, steps, warmup)
    scorer_ms, _ = _graph_time(fs.run_score_only, replicas, steps, warmup)
    select_ms, _ = _graph_time(fs.run_select, replicas, steps, warmup)
    attend_ms, _ = _graph_time(fs.run_attend, replicas, steps, warmup)
    select_attend_ms, _ = _graph_time(fs.run_select_attend, replicas, steps, warmup)
    torch.cuda.synchronize()
    sb = scorer_bytes(case)
    ab = []
    for i in range(replicas):
        sel = fs.sets[i][3].cpu().numpy()
        qh = case.q if i == 0 else case.replicas[i - 1][0]
        ab.append(step_bytes(case, qh, sel))
    att = sum(b["algorithmic"] for b in ab) / len(ab)
    eff = sum(b["effective_kv"] for b in ab) / len(ab)
    res = {
        "config": name, "steps": n, "steps_requested": steps, "ms_per_step": step_ms,
        "step_note": "two launches: the scorer (msa_block_score_topk, topk_out NULL), then "
                     "the attend that selects each row's top-16 itself "
                     "(msa_sparse_decode_select_run)",
        "ms_per_step_three_launches": separate_ms,
        "tokens_per_s": case.real_rows / (step_ms / 1e3),
        "scorer_ms": scorer_ms, "score_topk_ms": score_ms, "select_ms": select_ms,
        "attend_ms": attend_ms, "select_attend_ms": select_attend_ms,
        "score_k_half_bytes": sb["k_half"], "score_algorithmic_bytes": sb["algorithmic"],
        # the scorer alone (msa_block_score_topk with topk_out NULL)
        "scorer_bytes": sb["scorer"],
        "scorer_gbs": sb["scorer"] / (scorer_ms / 1e3) / 1e9,
        "scorer_pct_hbm_peak": 100 * sb["scorer"] / (scorer_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "score_traffic_bytes": (lambda t: None if t is None else t.get("hbm_bytes_per_launch"))(
            load_traffic(name, "score")),
        # MFMA use of the HBM-bound scorer: its matrix-core flops over its
        # time, against the dense peak of the MFMA it issues (bf16 q: bf16,
        # fp8 q: fp8).
        "scorer_mfma_tflops": sb["mfma_flops"] / (scorer_ms / 1e3) / 1e12,
        "scorer_mfma_peak_tflops": MFMA_PEAK_TFLOPS[case.q_dtype == "fp8_e4m3"],
        "scorer_mfma_pct_peak": 100 * sb["mfma_flops"] / (scorer_ms / 1e3) / 1e12
                                / MFMA_PEAK_TFLOPS[case.q_dtype == "fp8_e4m3"],
        "attend_algorithmic_bytes": att, "attend_effective_kv_bytes": eff,
        "attend_algorithmic_gbs": att / (attend_ms / 1e3) / 1e9,
        "step_algorithmic_gbs": (att + sb["algorithmic"]) / (step_ms / 1e3) / 1e9,
        "splits": fs.plan.num_splits, "real_rows": case.real_rows,
    }
    ts = scorer_ms / 1e3
    res["roofline"] = _roofline(
        sb["scorer"], sb["mfma_flops"], ts, MFMA_PEAK_TFLOPS[case.q_dtype == "fp8_e4m3"],
        res["score_traffic_bytes"],
        {"kernel": f"score_kernel<kv {case.kv_dtype}, q {case.q_dtype}>",
         "basis": "K half of every visible row of every (request, kv head) + q + the score "
                  "write + block-table entries",
         "timing": "HIP events: graph replays of the scorer alone"})
    uq = sum(b["unique_algorithmic"] for b in ab) / len(ab)
    fl = sum(b["flops"] for b in ab) / len(ab)
    at = load_traffic(name, "attend")
    res["attend_roofline"] = _roofline(
        uq, fl, attend_ms / 1e3, MFMA_PEAK_TFLOPS[False],
        None if at is None else at.get("hbm_bytes_per_launch"),
        {"kernel": f"attend_kernel<kv {case.kv_dtype}, q {case.q_dtype}>",
         "basis": UNIQUE_BASIS, "timing": "HIP events around graph replays of the attend"})
    # The attend of the two-launch step: the same pages plus one read of
    # every (token row, kv head) score row it selects from, and no top-k read.
    sa = load_traffic(name, "attend", record="select_attend")
    res["select_attend_roofline"] = _roofline(
        uq - sb["topk"] + sb["score_read"], fl, select_attend_ms / 1e3, MFMA_PEAK_TFLOPS[False],
        None if sa is None else sa.get("hbm_bytes_per_launch"),
        {"kernel": f"attend_kernel<kv {case.kv_dtype}, q {case.q_dtype}, selecting>",
         "basis": UNIQUE_BASIS + ", with the score rows it selects from in place of the "
                  "top-k entries",
         "timing": "HIP events around graph replays of the selecting attend"})
    res["step_pct_hbm_peak"] = 100 * res["step_algorithmic_gbs"] / HBM_PEAK_GBS
    del fs
    torch.cuda.empty_cache()
    return res


def _oracle_row(case, t: int):
    """The oracle on one token row of the case (all its kv heads)."""
    from oracle import msa_oracle as om

    if hasattr(case, "cu_seqlens_q"):
        return om.sparse_prefill(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                                 case.block_table, case.cu_seqlens_q, case.context_lens,
                                 case.topk, case.num_kv_heads, case.sm_scale, rows=[t],
                                 q_dtype=case.q_dtype, q_scale=case.q_scale)
    if case.topk is None:
        return om.dense_decode(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                               case.block_table, case.seq_lens, case.dql, case.num_kv_heads,
                               case.sm_scale, rows=[t], q_dtype=case.q_dtype,
                               q_scale=case.q_scale)
    return om.sparse_decode(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                            case.block_table, case.seq_lens, case.topk, case.dql,
                            case.num_kv_heads, case.sm_scale, rows=[t], q_dtype=case.q_dtype,
                            q_scale=case.q_scale)


def _oracle_full_step_row(case, t: int):
    """The oracle's full decode step for one token row: its block-max scores,
    their top-k, and the attend over that selection (all kv heads)."""
    import numpy as np

    from oracle import msa_oracle as om

    score = om.block_max_scores(case.q, case.kv, case.kv_dtype, case.k_scale, case.block_table,
                                case.seq_lens, case.dql, case.num_kv_heads, case.max_blocks,
                                rows=[t], q_dtype=case.q_dtype, q_scale=case.q_scale)
    topk = np.full((case.num_token_rows, case.num_kv_heads, case.topk_k), -1, dtype=np.int32)
    topk[t] = om.select_topk(score, case.topk_k)[0]
    return om.sparse_decode(case.q, case.kv, case.kv_dtype, case.k_scale, case.v_scale,
                            case.block_table, case.seq_lens, topk, case.dql, case.num_kv_heads,
                            case.sm_scale, rows=[t], q_dtype=case.q_dtype, q_scale=case.q_scale)


def oracle_full_step_rate(case, seconds: float):
    """Token rows per second of the oracle's full step (score -> top-k ->
    attend), one BLAS thread, over rows in a seeded order for about
    `seconds`; returns (rows done, rows per second)."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    order = np.random.default_rng(0).permutation(case.real_rows)
    done = 0
    t0 = time.perf_counter()
    try:
        for t in order:
            _oracle_full_step_row(case, int(t))
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return done, done / (time.perf_counter() - t0)


def _oracle_rows_for(case, order, seconds: float) -> int:
    """Rows of `order` (cycled) through the oracle for about `seconds`, with
    BLAS limited to one thread; returns the count done."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    done = 0
    t0 = time.perf_counter()
    try:
        while True:
            for t in order:
                _oracle_row(case, int(t))
                done += 1
                if time.perf_counter() - t0 >= seconds:
                    return done
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def cpu_baseline(case, seconds: float):
    """The float64 oracle, single-threaded, on a bounded sample of the same
    workload's token rows; scaled to tokens/s."""
    import numpy as np

    order = np.random.default_rng(0).permutation(case.real_rows)
    t0 = time.perf_counter()
    rows_done = _oracle_rows_for(case, order, seconds)
    el = time.perf_counter() - t0
    b = step_bytes(case, case.q, case.topk)
    per_row_bytes = b["effective_kv"] / case.real_rows
    return {
        "value": rows_done / el,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{rows_done} token rows (passes over the {case.real_rows} rows of "
                  f"replica 0 in a seeded order; {rows_done * case.num_kv_heads} "
                  f"(token, kv head) units), {el:.1f} s, one thread (BLAS limited to 1)",
        "effective_kv_gbs": rows_done * per_row_bytes / el / 1e9,
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_POOL_CASE = None


def _pool_worker(args):
    order, seconds = args
    return _oracle_rows_for(_POOL_CASE, order, seconds)


def cpu_pool_baseline(name: str, seconds: float, max_workers: int = 16):
    """The same oracle on every core of the host's share: the workload's rows
    dealt round-robin to a process pool (one BLAS thread each), each worker
    busy for about `seconds`.  Runs in a process that never touches the GPU
    (the bench starts it before its own GPU work)."""
    import multiprocessing as mp

    import numpy as np

    global _POOL_CASE
    _POOL_CASE = make_case(name, 0)
    case = _POOL_CASE
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    order = np.random.default_rng(0).permutation(case.real_rows)
    parts = [(order[i::workers], seconds) for i in range(workers)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        counts = pool.map(_pool_worker, parts)
    el = time.perf_counter() - t0
    rows_done = int(sum(counts))
    b = step_bytes(case, case.q, case.topk)
    per_row_bytes = b["effective_kv"] / case.real_rows
    return {
        "value": rows_done / el,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{rows_done} token rows of replica 0 dealt round-robin to {workers} "
                  f"worker processes (one BLAS thread each), {el:.1f} s wall",
        "effective_kv_gbs": rows_done * per_row_bytes / el / 1e9,
    }


def kernel_key(res) -> str:
    """The kernel family that runs a workload's attend: the single-row attend
    or the multi-row tile kernel."""
    return "attend" if res.get("tile_rows", 1) == 1 else "tile"


def traffic_path(config: str, kernel: str) -> str:
    return os.path.join(TRAFFIC_DIR, f"{kernel}_{config}_traffic.json")


def load_traffic(config: str, kernel: str, record: Optional[str] = None):
    """HBM bytes per launch of `kernel` on `config` from the committed
    rocprofv3 counter summary (file named for `record`, default the kernel's
    own name), if it was taken on the current sources of that kernel; else
    None."""
    try:
        with open(traffic_path(config, record or kernel)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha") != kernel_source_hash(kernel):
        return None
    return rec


UNIQUE_BASIS = ("unique K|V page rows (each distinct (request, kv head, page) once, at the "
                "largest visible count any of its token rows has) + q + out + top-k entries "
                "+ block-table entries, per attend launch: the least the launch must move "
                "from HBM")


def _roofline(bytes_per_launch, flops_per_launch, seconds, mfma_peak, traffic, extra):
    """A roofline record for one kernel launch: HBM rate against 8 TB/s and
    matrix-core rate against the dense MFMA peak; `bound`, `achieved`, `peak`
    and `frac` are the binding one (the larger fraction)."""
    gbs = bytes_per_launch / seconds / 1e9
    tflops = flops_per_launch / seconds / 1e12
    hbm_frac, mfma_frac = gbs / HBM_PEAK_GBS, tflops / mfma_peak
    hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(hbm_frac, 4)}
    mfma = {"achieved": round(tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s",
            "frac": round(mfma_frac, 4)}
    top = hbm if hbm_frac >= mfma_frac else mfma
    rec = {"bound": "hbm" if hbm_frac >= mfma_frac else "mfma", **top,
           "traffic": traffic, "hbm": hbm, "mfma": mfma,
           "bytes_per_launch": int(bytes_per_launch), "flops_per_launch": int(flops_per_launch),
           "avg_launch_us": round(seconds * 1e6, 3)}
    rec.update(extra)
    return rec


def attend_roofline(res, case):
    """The attend launch's roofline on unique bytes (see UNIQUE_BASIS), with
    the per-token (effective) rate beside it."""
    kernel = kernel_key(res)
    t = res["attend_ms"] / 1e3
    traffic = load_traffic(res["config"], kernel)
    label = (f"attend_kernel<kv {case.kv_dtype}, q {case.q_dtype}>" if kernel == "attend" else
             f"multi_kernel<kv {case.kv_dtype}, q {case.q_dtype}, rows {res['tile_rows']}>")
    return _roofline(
        res["unique_algorithmic_bytes"], res["attend_flops"], t, MFMA_PEAK_TFLOPS[False],
        None if traffic is None else traffic.get("hbm_bytes_per_launch"),
        {"kernel": label, "basis": UNIQUE_BASIS,
         "effective_gbs": round(res["algorithmic_bytes"] / t / 1e9, 1),
         "effective_note": "per-token logical bytes over the launch: pages shared by a "
                           "request's token rows count once per row, and the L2 / MALL serve "
                           "the repeats, so this is not an HBM bandwidth and can exceed 8 TB/s",
         "mfma_note": "attend flops = 4 * G * 128 per (visible key, token row, kv head); "
                      "bf16 dense peak (P V is a bf16 MFMA whatever the q format)",
         "timing": "HIP events around graph replays of the attend launches alone, on the "
                   "stream they run on",
         "traffic_source": None if traffic is None else traffic.get("source")})


def profile_mode(name, launches, splits, dev):
    """Eager launches of whole steps for rocprofv3 (kernel trace / counters)."""
    import torch

    from workloads import gen

    case = make_case(name, 1)
    if name == FULL_STEP_CONFIG:
        fs = FullStepSet(case, 2, dev)
        for i in range(launches):
            fs.run_step(i % 2)
        torch.cuda.synchronize()
        print(json.dumps({"profile_mode": name, "launches": launches,
                          "scorer_bytes_per_launch": scorer_bytes(case)["scorer"],
                          "selector_bytes_per_launch": scorer_bytes(case)["selector"],
                          "kernel_source_sha": kernel_source_hash("score")}), flush=True)
        return
    ds = DeviceSet(case, 2, splits, dev)
    for i in range(launches):
        ds.run_step(i % 2)
    torch.cuda.synchronize()
    b = ds.mean_bytes("algorithmic")
    print(json.dumps({"profile_mode": name, "launches": launches,
                      "algorithmic_bytes_per_launch": b,
                      "effective_kv_bytes_per_launch": ds.mean_bytes("effective_kv"),
                      "unique_kv_bytes_per_launch": ds.mean_bytes("unique_kv"),
                      "unique_algorithmic_bytes_per_launch": ds.mean_bytes("unique_algorithmic"),
                      "tile_rows": ds.plan.tile_rows, "splits": ds.plan.num_splits,
                      "kernel_source_sha": kernel_source_hash(
                          "attend" if ds.plan.tile_rows == 1 else "tile")}), flush=True)


def copy_calibration(dev, mib=1024, launches=4):
    """A plain device copy of known size: the FETCH_SIZE / WRITE_SIZE scale."""
    import torch

    n = mib * 2**20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(launches):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": launches}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", default=DEFAULT_CONFIG,
                    choices=sorted(k for k in CONFIG_TEXT if k != FULL_STEP_CONFIG))
    ap.add_argument("--full-step-only", action="store_true",
                    help="time only the full step with the indexer and print its record")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--splits", type=int, default=0, help="0 = the plan's choice")
    ap.add_argument("--tile-rows", type=int, default=0,
                    help="token rows per workgroup: 0 = the plan's choice, 1, 2 or 4")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--profile-mode", action="store_true")
    ap.add_argument("--profile-launches", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cpu-pool-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_pool_child:
        print(json.dumps(cpu_pool_baseline(args.config, args.cpu_seconds)), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested). The decode step shards by kv head or by "
              f"request with no exchange, so each GPU would run this same kernel on its "
              f"share.", file=sys.stderr)
        sys.exit(2)

    # The all-core oracle baseline runs in a child process started before this
    # process touches the GPU (a process pool must not be forked from one that
    # has).
    cpu_pool = None
    if not (args.no_cpu_baseline or args.profile_mode or args.copy_calibration
            or args.full_step_only):
        import subprocess

        try:
            child = subprocess.run(
                [sys.executable, os.path.abspath(__file__), "--cpu-pool-child", "--config",
                 args.config, "--cpu-seconds", str(args.cpu_seconds)],
                capture_output=True, text=True, timeout=args.cpu_seconds * 4 + 120)
            lines = [ln for ln in child.stdout.splitlines() if ln.startswith("{")]
            if child.returncode == 0 and lines:
                cpu_pool = json.loads(lines[-1])
            else:
                print(f"[bench] all-core oracle baseline failed: {child.stderr[-500:]}",
                      file=sys.stderr)
        except subprocess.TimeoutExpired:
            print("[bench] all-core oracle baseline timed out", file=sys.stderr)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    import block_sparse_gqa_decode_amd as msa

    msa.load_library()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.profile_mode:
        profile_mode(FULL_STEP_CONFIG if args.full_step_only else args.config,
                     args.profile_launches, args.splits, dev)
        return

    if args.full_step_only:
        r5 = time_full_step(FULL_STEP_CONFIG, max(32, args.steps // 8), args.warmup,
                            args.replicas, dev)
        print(json.dumps(r5), flush=True)
        return
    res, case = time_config(args.config, args.steps, args.warmup, args.replicas,
                            args.splits, dev, tile_rows=args.tile_rows, cold=True,
                            ceiling=True)
    others = {}
    if not args.no_other_configs:
        for name in OTHER_CONFIGS:
            if name == args.config:
                continue
            r2, case2 = time_config(name, args.steps, args.warmup,
                                    args.replicas, args.splits, dev,
                                    ceiling=name in ("c2_tp4_fp8", "c3_tp1_fp8"))
            r2["roofline"] = attend_roofline(r2, case2)
            if not args.no_cpu_baseline:
                # a short single-thread oracle sample beside each GPU number
                import numpy as np

                order = np.random.default_rng(0).permutation(case2.real_rows)
                t0 = time.perf_counter()
                n_rows = _oracle_rows_for(case2, order, 2.0)
                r2["oracle_tokens_per_s_1thread"] = n_rows / (time.perf_counter() - t0)
                r2["gpu_over_oracle"] = r2["tokens_per_s"] / r2["oracle_tokens_per_s_1thread"]
            others[name] = {k: (round(v, 4) if isinstance(v, float) else v)
                            for k, v in r2.items()}
        r5 = time_full_step(FULL_STEP_CONFIG, args.steps, args.warmup, args.replicas, dev)
        if not args.no_cpu_baseline:
            from workloads import gen

            n5, rate5 = oracle_full_step_rate(gen.make_config(FULL_STEP_CONFIG), 3.0)
            r5["oracle_tokens_per_s_1thread"] = rate5
            r5["oracle_sample"] = (f"{n5} token rows through the oracle's score -> top-16 -> "
                                   "attend, one thread")
            r5["gpu_over_oracle"] = r5["tokens_per_s"] / rate5
        others[FULL_STEP_CONFIG] = {k: (round(v, 4) if isinstance(v, float) else v)
                                    for k, v in r5.items()}
    roofline = attend_roofline(res, case)
    roofline["measured_ceiling"] = res.get("measured_ceiling")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "steps_requested": args.steps,
        "steps_note": f"timed steps = --steps rounded up to at least {MIN_TIMED_STEPS} steps and "
                      f"at least {MIN_TIMED_MS:.0f} ms of replays (at the warmup replays' rate), "
                      f"in whole cycles of the {args.replicas} replicas captured in one graph: "
                      f"the GPU runs its first ~30 ms after an idle spell up to 10% slower",
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {CONFIG_TEXT[args.config]}",
            "kv_cache": case.kv_dtype,
            "global_batch": case.batch,
            "decode_query_len": getattr(case, "dql", 0),
            "num_token_rows": case.num_token_rows,
            "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads,
            "topk_blocks": case.topk_k if case.topk is not None else "dense",
            "page_size": 128,
            "head_dim": 128,
            "replicas": args.replicas,
            "splits": res["splits"],
            "tile_rows": res["tile_rows"],
            "parallelism": "single GPU",
        },
        "effective_kv_gbs": round(res["effective_kv_gbs"], 1),
        "effective_kv_note": "per-token logical K|V bytes per step time; repeats of a page "
                             "across a request's token rows count each time (the L2 / MALL "
                             "serve them), so this is not an HBM bandwidth",
        "unique_kv_gbs": round(res["unique_kv_gbs"], 1),
        "unique_pct_hbm_peak": round(res["unique_pct_peak"], 2),
        "host_ms_per_step": round(res["host_ms_per_step"], 5),
        "cold_ms_per_step": round(res["cold_ms_per_step"], 5),
        "warm_ms_per_step": round(res["warm_ms_per_step"], 5),
        "cold_warm_note": "one step replayed alone as its own graph right after a 1 GiB "
                          "scrub write (cold) and again straight after (warm: pages in "
                          "L2/MALL), medians of 5, each including one graph launch; "
                          "cross-checks, not the value",
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_pool,
        "other_configs": others,
        "kernel_source_sha": {k: kernel_source_hash(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
