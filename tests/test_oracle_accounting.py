"""Pins of the oracle's accounting (CPU only).

 * visible pairs and the tree-token ratio of the worked example of the
   tree-training page (section 树构建过程: 8 tree tokens for 11 original ones,
   22 visible pairs read off the figure, tests/golden/worked_example.json);
 * attention FLOPs against torch's own FLOP counter
   (torch.utils.flop_counter.FlopCounterMode) run over attention written one
   query at a time with each query's visible keys gathered: the forward's
   products, and the backward's products plus the score product it
   recomputes from the saved row statistics;
 * the bench's FLOP count is the oracle's.
"""

import json
import os

import numpy as np
import pytest
import torch
from torch.utils.flop_counter import FlopCounterMode

import oracle
from workloads import worked_example

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_worked_example_counts():
    g = json.load(open(GOLDEN))
    f = oracle.build_forest(worked_example(), g["max_tokens_per_mb"])
    st = oracle.forest_stats(f, worked_example())
    assert st["pairs"] == g["n_pairs"] == 22
    assert st["causal_pairs"] == g["causal_pairs"] == 26
    assert st["tree_tokens"] == 8 and st["orig_tokens"] == 11
    assert st["tree_token_ratio"] == pytest.approx(8 / 11, abs=0)


def _counted(tree, hq, hkv, d, seed):
    """(forward FLOPs, backward FLOPs incl. the recomputed scores) that torch
    counts for attention over each real query's gathered ancestors."""
    rng = np.random.default_rng(seed)
    N = tree.n_tokens
    G = hq // hkv
    q = torch.tensor(rng.standard_normal((N, hq, d)), requires_grad=True)
    k = torch.tensor(rng.standard_normal((N, hkv, d)), requires_grad=True)
    v = torch.tensor(rng.standard_normal((N, hkv, d)), requires_grad=True)
    with FlopCounterMode(display=False) as fwd:
        outs = []
        for i in range(N):
            anc = torch.as_tensor(oracle.ancestors(tree, i))
            for h in range(hq):
                kk, vv = k[anc, h // G], v[anc, h // G]          # [n_i, d]
                s = (kk @ q[i, h][:, None]).T / np.sqrt(d)       # [1, n_i]
                outs.append(torch.softmax(s, -1) @ vv)           # [1, d]
        loss = sum((o * o).sum() for o in outs)
    with FlopCounterMode(display=False) as bwd:
        loss.backward()
    with FlopCounterMode(display=False) as rec:   # the backward's recomputed Q.K^T
        with torch.no_grad():
            for i in range(N):
                anc = torch.as_tensor(oracle.ancestors(tree, i))
                for h in range(hq):
                    _ = k[anc, h // G] @ q[i, h][:, None]
    return fwd.get_total_flops(), bwd.get_total_flops() + rec.get_total_flops()


@pytest.mark.parametrize("seqs,cap,hq,hkv,d", [
    (worked_example(), 128, 2, 1, 64),
    (worked_example(), 128, 4, 2, 16),
    ([np.array([1, 2, 3, 4, 5, 6], np.int32), np.array([1, 2, 3, 9], np.int32),
      np.array([8, 8], np.int32)], 128, 3, 3, 8),
])
def test_attn_flops_match_torch_counter(seqs, cap, hq, hkv, d):
    tree = oracle.build_forest(seqs, cap).trees[0]
    fl = oracle.attn_flops(tree.n_pairs, hq, d)
    fwd, bwd = _counted(tree, hq, hkv, d, 3)
    assert fl["fwd"] == fwd
    assert fl["bwd"] == bwd
    assert fl["fwd_bwd"] == fwd + bwd


def test_bench_uses_the_oracle_flop_count():
    import bench
    for pairs, hq, d in ((22, 2, 64), (17_630_000, 32, 128), (123_456_789, 40, 128)):
        assert bench.attn_flops(pairs, hq, d) == oracle.attn_flops(pairs, hq, d)
