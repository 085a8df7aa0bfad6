"""Host-side checks of the benchmark (no GPU needed).

The benchmark counts the work it divides by time with its own closed forms
(it does not call the oracle on the timed path); these must agree with the
oracle's explicit masks.  It must refuse runs on more than one GPU.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import ksa_oracle as O  # noqa: E402


@pytest.mark.parametrize("n,k,C", [(1, 1, 0), (7, 8, 2), (37, 8, 2), (45, 4, 3), (101, 8, 3), (96, 3, 40),
                                   (64, 1, 5), (200, 8, 0)])
def test_visible_pairs_match_oracle_mask(n, k, C):
    assert bench.visible_pairs(n, k, C) == int(O.visibility_mask(n, k, C).sum())


def test_visible_pairs_of_the_timed_workloads():
    # pinned by the oracle's closed form, itself checked against brute force
    for n, k, C in [(32768, 8, 64), (131072, 8, 64), (131072, 8, 16), (8192, 8, 64)]:
        assert bench.visible_pairs(n, k, C) == O.visible_pairs_general(n, k, C)


@pytest.mark.parametrize("n,k,C,W", [(37, 8, 2, 5), (45, 4, 3, 1), (101, 8, 3, 40), (20, 3, 0, 100)])
def test_baseline_pairs_match_oracle_masks(n, k, C, W):
    assert bench.baseline_pairs(n, k, O.MODE_SCA, C, W) == int(O.baseline_mask(n, k, O.MODE_SCA, C=C).sum())
    assert bench.baseline_pairs(n, k, O.MODE_SWA, C, W) == int(O.baseline_mask(n, k, O.MODE_SWA, W=W).sum())


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2
