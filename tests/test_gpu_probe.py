"""GPU check of the memory-rate probe msa_probe_read_runs: every workgroup's
XOR of the 32-bit words of its runs, and its count of skipped runs, are
compared bit-exactly with numpy over the same bytes.  The cases cover runs
of every size class (16 bytes, partial and whole 32 KiB pages), empty
workgroups, odd run counts (the ring's tail), runs that must be skipped
(misaligned, empty, too long, outside the buffer) and a workgroup past the
512-run limit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _expected(buf, offs, lens, ranges, max_runs=512):
    """ranges[w] = (first, last) run of workgroup w, already clamped."""
    words = buf.view(np.uint32)
    x = np.zeros(len(ranges), dtype=np.uint32)
    bad = np.zeros(len(ranges), dtype=np.uint32)
    for w, (lo, hi) in enumerate(ranges):
        if hi - lo > max_runs:
            bad[w] += hi - lo - max_runs
            hi = lo + max_runs
        for i in range(lo, hi):
            o, n = int(offs[i]), int(lens[i])
            if o < 0 or n < 16 or n > 32768 or n % 16 or o % 16 or o + n > buf.nbytes:
                bad[w] += 1
                continue
            x[w] ^= np.bitwise_xor.reduce(words[o // 4:(o + n) // 4])
    return x, bad


def _run(buf, offs, lens, first):
    import torch

    import block_sparse_gqa_decode_amd as msa

    dev = torch.device("cuda:0")
    b = torch.from_numpy(buf).to(dev)
    out = torch.full((2 * (len(first) - 1),), -1, dtype=torch.int32, device=dev)
    msa.msa_probe_read_runs(b, torch.from_numpy(offs).to(dev), torch.from_numpy(lens).to(dev),
                            torch.from_numpy(first).to(dev), out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    return o[0::2], o[1::2]


def test_probe_checksums_match_numpy():
    print("[case] read-runs probe: 300 workgroups of random runs over 16 MiB", flush=True)
    rng = np.random.default_rng(11)
    buf = rng.integers(0, 256, size=16 << 20, dtype=np.uint8)
    counts = rng.integers(0, 12, size=300)
    counts[7] = 0
    counts[8] = 1
    counts[9] = 530          # past the per-workgroup limit
    first = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(first[-1])
    lens = (rng.integers(1, 2049, size=n) * 16).astype(np.int32)
    lens[rng.random(n) < 0.3] = 32768
    offs = (rng.integers(0, (buf.nbytes - 32768) // 16, size=n) * 16).astype(np.int64)
    # Runs the kernel must skip, and count.
    bad_idx = rng.choice(n, size=40, replace=False)
    kinds = np.arange(40) % 5
    offs[bad_idx[kinds == 0]] += 8                       # misaligned
    lens[bad_idx[kinds == 1]] = 0                        # empty
    lens[bad_idx[kinds == 2]] = 32768 + 16               # longer than a page
    offs[bad_idx[kinds == 3]] = buf.nbytes - 16 * 5      # runs past the end
    lens[bad_idx[kinds == 3]] = 16 * 6
    offs[bad_idx[kinds == 4]] = -4096                    # before the start
    x, bad = _run(buf, offs, lens, first)
    ex, ebad = _expected(buf, offs, lens, list(zip(first[:-1], first[1:])))
    assert np.array_equal(bad, ebad)
    assert np.array_equal(x, ex)
    assert ebad.sum() >= 40 + (530 - 512)


def test_probe_clamps_workgroup_ranges():
    print("[case] read-runs probe: out-of-order and out-of-range run ranges", flush=True)
    rng = np.random.default_rng(12)
    buf = rng.integers(0, 256, size=1 << 20, dtype=np.uint8)
    offs = (np.arange(8) * 32768).astype(np.int64)
    lens = np.full(8, 32768, dtype=np.int32)
    # Each workgroup's range is clamped into [0, 8] on its own: a decreasing
    # one reads nothing, one past the end stops at run 8.
    first = np.array([0, 3, 2, 8, 12], dtype=np.int32)
    x, bad = _run(buf, offs, lens, first)
    ex, ebad = _expected(buf, offs, lens, [(0, 3), (3, 3), (2, 8), (8, 8)])
    assert np.array_equal(x, ex) and np.array_equal(bad, ebad)
    assert x[1] == 0 and x[3] == 0
