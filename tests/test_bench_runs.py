"""Host checks of the byte runs that bench.py feeds the memory-rate probe
(no GPU): for the attend's own launch layout they must cover exactly the
effective K|V bytes of the step (the visible rows of every live page of every
(token, kv head)), in bounds and aligned; the
contiguous variant must read the same bytes per workgroup."""
import types

import numpy as np
import pytest
import torch

import bench
from workloads import gen


def _fake_ds(case, splits):
    kv = bench._host_kv(case)
    bt = torch.from_numpy(case.block_table)
    return types.SimpleNamespace(case=case, kv=kv, steps=[(None, bt, None, None)],
                                 plan=types.SimpleNamespace(num_splits=splits))


@pytest.mark.parametrize("name,splits", [("c1_tiny_bf16", 1), ("c1_tiny_bf16", 4),
                                         ("c2_tp4_fp8", 2), ("c2_tp4_fp8", 3)])
def test_page_runs_cover_the_effective_bytes(name, splits):
    case = gen.make_config(name)
    ds = _fake_ds(case, splits)
    offs, lens, first = bench.attend_page_runs(ds, 0)
    eff = bench.step_bytes(case, case.q, case.topk)["effective_kv"]
    assert int(lens.astype(np.int64).sum()) == eff
    nbytes = ds.kv.numel() * ds.kv.element_size()
    assert (offs % 16 == 0).all() and (lens % 16 == 0).all()
    assert (lens >= 16).all() and (lens <= 32768).all()
    assert (offs >= 0).all() and (offs + lens <= nbytes).all()
    assert np.all(np.diff(first) >= 0) and first[-1] == len(offs)
    assert np.diff(first).max() <= 512
    co, cl, cf = bench.contiguous_runs(lens, first, 0, nbytes)
    assert len(cf) == len(first)
    for w in range(len(first) - 1):
        assert cl[cf[w]:cf[w + 1]].astype(np.int64).sum() == \
            lens[first[w]:first[w + 1]].astype(np.int64).sum()
    assert (co % 16 == 0).all() and (co + cl <= nbytes).all()


def test_timed_window_rule():
    """Timed windows: --steps rounded up to at least MIN_TIMED_STEPS steps and
    to MIN_TIMED_MS of replays, in whole replays of the replicas."""
    r = 8
    # a slow step: the step count decides (200 steps = 25 replays of 8)
    assert bench.window_replays(1000.0, 20, r) == (bench.MIN_TIMED_STEPS + r - 1) // r
    # more steps asked than the floor: rounded up to whole replays
    assert bench.window_replays(1000.0, 1001, r) == 126
    # a fast step: the duration decides
    n = bench.window_replays(0.65, 20, r)
    assert n * 0.65 >= bench.MIN_TIMED_MS and (n - 1) * 0.65 < bench.MIN_TIMED_MS
    # a degenerate timing never gives an unbounded window
    assert bench.window_replays(0.0, 20, r) == 200000
