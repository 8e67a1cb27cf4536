"""Host allocation of libpst (FFD, Karmarkar-Karp, metrics) against the
oracle, item by item (CPU only: these entry points never touch the GPU).

Inputs: seeded random weights (spanning ties, zeros, single items, groups
beyond the item count), the packing page's bimodal length mix, and the
per-tree attention-pair counts of the bimodal workload's forest as built by
the oracle.  Group assignments and fallback flags must match exactly;
metrics to float rounding.
"""

import random

import numpy as np
import pytest

import oracle
import prefix_shared_tree_packed_amd as pst
from oracle import packing
from prefix_shared_tree_packed_amd import _lib
from workloads import bimodal_lengths, get_workload


def _as_group_of(groups, n):
    g = np.full(n, -1, dtype=np.int64)
    for j, items in enumerate(groups):
        g[list(items)] = j
    return g


def _compare(values, capacity, min_groups, divisor, algorithm):
    ref_groups, ref_fb = packing.allocate(values, capacity, min_groups, divisor, algorithm)
    got_groups, got_fb = pst.pack_allocate(values, capacity, min_groups, divisor, algorithm)
    n = len(values)
    assert got_fb == ref_fb
    assert len(got_groups) == len(ref_groups)
    np.testing.assert_array_equal(_as_group_of(got_groups, n), _as_group_of(ref_groups, n))
    ref_m = packing.packing_metrics(values, ref_groups, capacity)
    got_m = pst.packing_metrics(values, got_groups, capacity)
    for key, ref in ref_m.items():
        assert got_m[key] == pytest.approx(ref, rel=1e-12, abs=1e-9), key


@pytest.mark.parametrize("algorithm", ["ffd", "kk"])
def test_random(algorithm):
    rng = random.Random(7 if algorithm == "ffd" else 8)
    for _ in range(300):
        n = rng.randint(1, 80)
        hi = rng.choice([1, 5, 100, 5000])
        values = [rng.randint(0, hi) for _ in range(n)]
        capacity = max(values) + rng.choice([0, 1, hi, 10 * hi, 10 ** 12])
        capacity = max(capacity, 1)
        _compare(values, capacity, rng.randint(1, 12), rng.choice([1, 1, 2, 3, 4]), algorithm)


@pytest.mark.parametrize("algorithm", ["ffd", "kk"])
@pytest.mark.parametrize("n,ranks", [(256, 4), (1024, 8), (4096, 4)])
def test_bimodal_lengths(algorithm, n, ranks):
    values = bimodal_lengths(n, seed=n + ranks).tolist()
    # micro-batches of 8192 tokens, and a pure balance over the ranks
    _compare(values, 8192, ranks, 1, algorithm)
    _compare(values, 10 ** 12, ranks, 1, algorithm)


def test_assign_trees_bimodal():
    w = get_workload("bimodal")
    ref_forest = oracle.build_forest(w.seqs, w.max_tokens_per_mb)
    forest = pst.build_tree(w.seqs, w.max_tokens_per_mb)
    for cost, attr in (("pairs", "n_pairs"), ("tokens", "n_tokens")):
        costs = [getattr(t, attr) for t in ref_forest.trees]
        for ranks in (2, 4, 8, 64):
            for algorithm in ("ffd", "kk"):
                ref_groups, _ = packing.allocate(costs, max(sum(costs), 1), ranks, 1, algorithm)
                got = pst.assign_trees(forest, ranks, cost=cost, algorithm=algorithm)
                np.testing.assert_array_equal(got, _as_group_of(ref_groups, len(costs)))


def test_errors():
    with pytest.raises(ValueError, match="ffd.*kk"):
        pst.pack_allocate([1, 2], 8, algorithm="lpt")
    with pytest.raises(pst.PstError) as e:
        pst.pack_allocate([5, 9], 8, algorithm="kk")
    assert "PST_ECAPACITY" in str(e.value)
    lib = pst.load()
    v = np.array([1, 2], dtype=np.int64)
    g = np.zeros(2, dtype=np.int32)
    ng = np.zeros(1, dtype=np.int32)
    args = (v.ctypes.data_as(_lib.P64), 2)
    out = (g.ctypes.data_as(_lib.P32), ng.ctypes.data_as(_lib.P32), None)
    assert _lib.ERRORS[lib.pst_pack_allocate(*args, 8, 1, 1, 7, *out)] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_pack_allocate(*args, 0, 1, 1, 0, *out)] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_pack_allocate(*args, 8, 0, 1, 0, *out)] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_pack_allocate(v.ctypes.data_as(_lib.P64), 0, 8, 1, 1, 0, *out)] \
        == "PST_EINVAL"
    neg = np.array([1, -2], dtype=np.int64)
    assert _lib.ERRORS[lib.pst_pack_allocate(neg.ctypes.data_as(_lib.P64), 2, 8, 1, 1, 1, *out)] \
        == "PST_EINVAL"
    bad = np.array([0, 3], dtype=np.int32)
    m = _lib.PackMetrics()
    import ctypes
    assert _lib.ERRORS[lib.pst_pack_metrics_compute(*args, bad.ctypes.data_as(_lib.P32), 2, 8,
                                                    ctypes.byref(m))] == "PST_ERANGE"
