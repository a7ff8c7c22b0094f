"""Host-side pieces of bench.py: the algorithmic byte count (valid rows,
window, custom mask) and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kept_rows():
    lens = [5, 0, 3]
    assert list(bench.kept_rows(lens)) == [5, 0, 3]
    assert list(bench.kept_rows(lens, window=2)) == [2, 0, 2]
    keep = np.array([1, 0, 1, 1, 0] + [] + [0, 1, 1], dtype=bool)
    assert list(bench.kept_rows(lens, keep=keep)) == [3, 0, 2]
    # a row must pass both: the window keeps rows 3, 4 of request 0 and 1, 2 of request 2
    assert list(bench.kept_rows(lens, window=2, keep=keep)) == [1, 0, 2]


def test_algorithmic_bytes_paged():
    p = W.make_paged("t", "bf16", 3, 8, 2, 64, 16, 5, lens=np.array([5, 0, 40]))
    es, row = 2, 2 * 64 * 2 * 2  # K and V of one row, all KV heads
    fixed = 2 * 3 * 8 * 64 * es + 4 * 3 * 8 + 4 * (p.total_used_pages + 2 * 3 + 1)
    assert bench.algorithmic_bytes(p) == 45 * row + fixed
    assert bench.algorithmic_bytes(p, window=10) == 15 * row + fixed
    keep = np.zeros(45, dtype=bool)
    keep[[0, 7, 44]] = True
    assert bench.algorithmic_bytes(p, keep=keep) == 3 * row + fixed


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_block_sparse_mask_runs():
    """random_mask(blocks=R): runs of exactly R rows kept or dropped together
    (the last run cut at the total), seeded, with about the asked share kept."""
    lens = [1000, 37, 2600]
    keep = W.random_mask(21, lens, keep=0.3, blocks=64)
    assert keep.shape == (3637,) and keep.dtype == bool
    runs = keep[: 3637 // 64 * 64].reshape(-1, 64)
    assert (runs.all(axis=1) | ~runs.any(axis=1)).all()  # every run uniform
    tail = keep[3637 // 64 * 64:]
    assert tail.all() or not tail.any()
    assert 0.15 < keep.mean() < 0.45
    assert np.array_equal(keep, W.random_mask(21, lens, keep=0.3, blocks=64))
    # runs of 1-40 rows (blocks=True) and independent rows stay as they were
    assert W.random_mask(21, lens, keep=0.3, blocks=True).shape == (3637,)
    assert W.random_mask(21, lens, keep=0.3).shape == (3637,)
