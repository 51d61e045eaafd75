"""Host-side logic of bench.py (no GPU): bucket splitting and the --gpus
contract."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("seed", range(5))
def test_bucket_runs_cover_every_chunk_once(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 2049, int(rng.integers(1, 400)))
    for bp in (1, 100, 2048, 5000, 10**6):
        runs = bench.bucket_runs(lens, bp)
        covered = np.concatenate([np.arange(f, f + c) for f, c in runs])
        assert np.array_equal(covered, np.arange(len(lens)))
        sizes = [int(lens[f:f + c].sum()) for f, c in runs]
        assert all(sz >= bp for sz in sizes[:-1])
        # whole chunks, no bucket one chunk longer than needed
        for (f, c), sz in zip(runs[:-1], sizes[:-1]):
            assert int(lens[f:f + c - 1].sum()) < bp


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
