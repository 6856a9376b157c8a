"""GPU run of the plain C consumer of the C ABI (tests/host/c_abi_decode.c):
one sparse decode step on device buffers from hipMalloc, through
msa_sparse_decode_plan / _run / _plan_destroy with no Python in between,
under the plan's own split choice, 2 splits merged in the attend and 8 splits
with the merge launch.  The program checks closed forms of the definition
(every visible V row equal gives that row times v_scale; padding rows and a
row with no selection give exact zeros; NaN past seq_len and on a spare page
never leaks) and exits 0 with "c-abi decode ok"."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu


def test_c_consumer_runs_a_decode_step():
    from block_sparse_gqa_decode_amd import build_lib

    exe = build_lib.C_CONSUMER_BIN
    assert os.path.exists(exe), "build() builds the C consumer beside the library"
    print("[case] C ABI consumer: decode step under 3 split plans", flush=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, (res.returncode, res.stdout, res.stderr)
    assert res.stdout.strip().splitlines()[-1] == "c-abi decode ok"
