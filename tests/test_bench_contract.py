"""Host-side parts of bench.py (CPU only): the one-GPU guard, and the count
of non-empty 32x32 blocks behind the reported block utilisation, checked
against the oracle's dense ancestor mask."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle.attention as oatt
import oracle.tree as otree
from workloads import get_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


@pytest.mark.parametrize("cap", [128, 256])
def test_block_count_matches_dense_mask(cap):
    sys.path.insert(0, ROOT)
    import bench
    import prefix_shared_tree_packed_amd as pst

    seqs = get_workload("tiny").seqs
    want = 0
    for t in otree.build_forest(seqs, cap).trees:
        M = oatt.dense_mask(t)
        nb = t.n_padded // 32
        want += int(M.reshape(nb, 32, nb, 32).any(axis=(1, 3)).sum())
    assert bench.blocks32(pst.build_tree(seqs, cap)) == want
