"""Oracle: micro-batch / rank allocation by FFD and Karmarkar-Karp, and the
packing-quality metrics (test infrastructure only).

Follows the article on AReaL's FFD and KK micro-batch packing (sections on
FFD, on KK with its implementation details and safety net, and on packing
quality metrics).  Readings where the article leaves a step open:

- FFD: items in stable descending order of value; while fewer groups than
  min_groups exist a new group is opened; otherwise the item goes to the
  lightest group that still has room (ties: lowest group index), else to a
  new group.  If the group count is not a multiple of the divisor, min_groups
  is raised to the next multiple and the packing redone; the count never
  exceeds the number of items (one item per group at most is forced).
- KK (largest differencing, k-way): every item starts as a state of k sets,
  the item alone in one of them.  The state with the largest spread
  (heaviest minus lightest set) and the next one are popped and merged by
  pairing the i-th lightest set of the first with the i-th heaviest set of
  the second; the result is pushed back, until one state is left.  Ties of
  spread: the state pushed first pops first.  Sets are kept in ascending
  order of sum (stable), and the final state's order numbers the groups.
- KK group count: max(min_groups, ceil(total / capacity)), rounded up to a
  multiple of the divisor, at most the number of items.  If a KK group still
  exceeds the capacity, the allocation falls back to FFD.
- An item larger than the capacity is an error.
- Metrics over the group sums s_g (G groups, total T, mean m = T / G):
  spread = max - min, imbalance_ratio = max / m, std_dev = population
  standard deviation, cv = std_dev / m (imbalance 1 and cv 0 when m = 0),
  utilization = T / (G * capacity), wasted_tokens = G * capacity - T.
"""

from __future__ import annotations

import heapq
import math


class CapacityError(ValueError):
    pass


def _check(values, capacity):
    if capacity <= 0:
        raise ValueError("capacity must be positive")
    for v in values:
        if v < 0:
            raise ValueError("values must be non-negative")
        if v > capacity:
            raise CapacityError(f"item of size {v} exceeds the capacity {capacity}")


def _ffd_once(values, capacity, min_groups):
    order = sorted(range(len(values)), key=lambda i: -values[i])  # stable
    sums, groups = [], []
    for i in order:
        v = values[i]
        if len(groups) < min_groups:
            sums.append(v)
            groups.append([i])
            continue
        best = -1
        for g in range(len(groups)):
            if sums[g] + v <= capacity and (best < 0 or sums[g] < sums[best]):
                best = g
        if best < 0:
            sums.append(v)
            groups.append([i])
        else:
            sums[best] += v
            groups[best].append(i)
    return groups


def ffd_allocate(values, capacity, min_groups=1, divisor=1):
    """Lists of item indices, one list per group (in creation order)."""
    values = [int(v) for v in values]
    _check(values, capacity)
    if not values:
        raise ValueError("no items")
    n = len(values)
    mg = max(1, min(min_groups, n))
    while True:
        groups = _ffd_once(values, capacity, mg)
        g = len(groups)
        if g % divisor == 0:
            return groups
        nxt = -(-g // divisor) * divisor
        if nxt > n:
            return groups
        mg = nxt


def kk_partition(values, k):
    """k-way largest differencing.  Returns k lists of item indices, in
    ascending order of their sums (ties in the order the merge produced)."""
    values = [int(v) for v in values]
    heap = []
    counter = 0
    for i, v in enumerate(values):
        sets = [(0, []) for _ in range(k - 1)] + [(v, [i])]
        heapq.heappush(heap, (-(v if k > 1 else 0), counter, sets))
        counter += 1
    while len(heap) > 1:
        _, _, a = heapq.heappop(heap)
        _, _, b = heapq.heappop(heap)
        merged = [(a[i][0] + b[k - 1 - i][0], a[i][1] + b[k - 1 - i][1]) for i in range(k)]
        merged.sort(key=lambda s: s[0])  # stable
        spread = merged[-1][0] - merged[0][0]
        heapq.heappush(heap, (-spread, counter, merged))
        counter += 1
    _, _, final = heap[0]
    return [items for _, items in final]


def kk_allocate(values, capacity, min_groups=1, divisor=1):
    """Returns (groups, fell_back)."""
    values = [int(v) for v in values]
    _check(values, capacity)
    if not values:
        raise ValueError("no items")
    n = len(values)
    total = sum(values)
    k = max(min_groups, -(-total // capacity), 1)
    k = -(-k // divisor) * divisor
    k = min(k, n)
    groups = kk_partition(values, k)
    if any(sum(values[i] for i in g) > capacity for g in groups):
        return ffd_allocate(values, capacity, min_groups, divisor), True
    return groups, False


def allocate(values, capacity, min_groups=1, divisor=1, algorithm="ffd"):
    if algorithm == "ffd":
        return ffd_allocate(values, capacity, min_groups, divisor), False
    if algorithm == "kk":
        return kk_allocate(values, capacity, min_groups, divisor)
    raise ValueError(f"unknown packing algorithm {algorithm!r}; valid: 'ffd', 'kk'")


def packing_metrics(values, groups, capacity):
    sums = [sum(int(values[i]) for i in g) for g in groups]
    G = len(sums)
    T = sum(sums)
    m = T / G
    var = sum((s - m) ** 2 for s in sums) / G
    std = math.sqrt(var)
    return {
        "n_groups": G,
        "total": T,
        "max_load": max(sums),
        "min_load": min(sums),
        "spread": max(sums) - min(sums),
        "imbalance_ratio": max(sums) / m if m > 0 else 1.0,
        "std_dev": std,
        "cv": std / m if m > 0 else 0.0,
        "utilization": T / (G * capacity),
        "wasted_tokens": G * capacity - T,
    }
