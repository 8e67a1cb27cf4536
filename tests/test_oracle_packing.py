"""Pins of the oracle's FFD / Karmarkar-Karp allocation and packing metrics
(CPU only).

 * two-way KK on 8, 7, 6, 5, 4 ends with sums 14 and 16 (difference 2, the
   textbook example of the differencing method, whose optimum is 0);
 * two-way KK's final difference equals that of the classic form of the
   method (replace the two largest numbers by their difference until one is
   left), on random inputs;
 * k-way KK: each merge keeps the spread within the larger of its two
   inputs' spreads, so the final spread never exceeds the largest item (a
   largest-with-largest pairing breaks this); every item lands in exactly
   one of k groups;
 * a three-way case traced by hand (9, 7, 6, 5, 4, 3 -> 11, 11, 12), which
   brute force shows is optimal;
 * FFD, the group-count rule and the KK -> FFD safety net on hand-worked
   cases; metrics of a hand-worked allocation.
"""

import itertools
import math
import random

import pytest

from oracle import packing


def _sums(values, groups):
    return [sum(values[i] for i in g) for g in groups]


def _classic_difference(values):
    xs = sorted(values)
    while len(xs) > 1:
        a = xs.pop()
        b = xs.pop()
        xs.append(a - b)
        xs.sort()
    return xs[0]


def _valid(values, groups, k):
    assert len(groups) == k
    seen = sorted(i for g in groups for i in g)
    assert seen == list(range(len(values)))


def test_kk_two_way_textbook():
    v = [8, 7, 6, 5, 4]
    groups = packing.kk_partition(v, 2)
    _valid(v, groups, 2)
    assert _sums(v, groups) == [14, 16]


def test_kk_two_way_matches_classic_differencing():
    rng = random.Random(3)
    for _ in range(200):
        v = [rng.randint(0, 1000) for _ in range(rng.randint(1, 40))]
        groups = packing.kk_partition(v, 2)
        _valid(v, groups, 2)
        s = _sums(v, groups)
        assert s[1] - s[0] == _classic_difference(v)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 7])
def test_kk_spread_bound_and_validity(k):
    rng = random.Random(10 + k)
    for _ in range(100):
        v = [rng.randint(0, 5000) for _ in range(rng.randint(1, 60))]
        groups = packing.kk_partition(v, k)
        _valid(v, groups, k)
        s = _sums(v, groups)
        assert s == sorted(s)
        assert s[-1] - s[0] <= max(v)


def test_kk_three_way_hand_trace_is_optimal():
    v = [9, 7, 6, 5, 4, 3]
    groups = packing.kk_partition(v, 3)
    assert [sorted(v[i] for i in g) for g in groups] == [[5, 6], [4, 7], [3, 9]]
    best = min(max(s) - min(s) for s in (
        [sum(x for x, a in zip(v, asg) if a == g) for g in range(3)]
        for asg in itertools.product(range(3), repeat=len(v))))
    assert best == 1 and _sums(v, groups)[-1] - _sums(v, groups)[0] == 1


def test_ffd_hand_cases():
    v = [5, 4, 3, 3, 2, 1]
    # 5 -> g0; 4 -> g1; 3 -> lighter of g0/g1 that fits (g1); 3 -> g0;
    # 2 fits nowhere -> g2; 1 -> lightest that fits (g2)
    assert packing.ffd_allocate(v, 8) == [[0, 3], [1, 2], [4, 5]]
    # 3 groups with divisor 2 -> min_groups 4: 5, 4, 3, 3 open groups; 2 goes
    # to the first of the two lightest (g2), 1 to g3
    assert packing.ffd_allocate(v, 8, divisor=2) == [[0], [1], [2, 4], [3, 5]]
    assert packing.ffd_allocate([1, 1, 1], 10, min_groups=2) == [[0, 2], [1]]
    # min_groups beyond the item count: one item per group
    assert packing.ffd_allocate([1, 1], 10, min_groups=5) == [[0], [1]]


def test_kk_allocate_group_count_and_safety_net():
    v = [10, 20, 30, 20, 20]
    # ceil(100 / 30) = 4, min 2 -> 4, multiple of 3 -> 6, at most 5 items
    groups, fb = packing.kk_allocate(v, 30, min_groups=2, divisor=3)
    assert not fb and len(groups) == 5
    # 3, 3, 2, 2, 2 into ceil(12 / 4) = 3 groups cannot fit capacity 4: KK
    # ends at 3 / 4 / 5, so FFD takes over and opens a fourth group
    groups, fb = packing.kk_allocate([3, 3, 2, 2, 2], 4)
    assert fb and groups == [[0], [1], [2, 3], [4]]
    assert packing.allocate([3, 3, 2, 2, 2], 4, algorithm="kk")[1]


def test_errors():
    with pytest.raises(packing.CapacityError):
        packing.ffd_allocate([5, 9], 8)
    with pytest.raises(packing.CapacityError):
        packing.kk_allocate([5, 9], 8)
    with pytest.raises(ValueError, match="ffd.*kk"):
        packing.allocate([1], 8, algorithm="lpt")


def test_metrics_hand():
    v = [5, 4, 3, 3, 2, 1]
    m = packing.packing_metrics(v, [[0, 3], [1, 2], [4, 5]], 8)
    assert (m["n_groups"], m["total"], m["max_load"], m["min_load"], m["spread"]) == (3, 18, 8, 3, 5)
    assert m["imbalance_ratio"] == pytest.approx(8 / 6)
    assert m["std_dev"] == pytest.approx(math.sqrt(14 / 3))
    assert m["cv"] == pytest.approx(math.sqrt(14 / 3) / 6)
    assert m["utilization"] == pytest.approx(0.75)
    assert m["wasted_tokens"] == 6
