"""Pins of the oracle's trie packing against what the pages and plain
combinatorics fix (CPU only).

 * the worked example of the tree-training page, read off its figure by hand;
 * hand-worked first-fit-decreasing cases;
 * brute force on many tiny random sequence sets: the packed tokens of a tree
   are exactly the distinct non-empty prefixes of its sequences, the ancestor
   relation is exactly "prefix of", sequences are recovered from their index
   maps, the capacity is never exceeded, tile classes agree with a scan of the
   dense mask.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.tree import BLOCK

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _check_nodes(tree, gold_nodes):
    assert len(tree.nodes) == len(gold_nodes)
    for n, g in zip(tree.nodes, gold_nodes):
        assert n.tokens == g["tokens"]
        assert (n.start_idx, n.end_idx) == (g["start_idx"], g["end_idx"])
        assert n.sequence_ids == g["sequence_ids"]
        assert n.children == {int(k): v for k, v in g["children"].items()}
        assert n.ancestors == g["ancestors"]


def test_worked_example():
    g = _load("worked_example.json")
    f = oracle.build_forest(g["seqs"], g["max_tokens_per_mb"])
    assert len(f.trees) == g["n_trees"]
    t = f.trees[0]
    assert t.n_tokens == g["n_tokens"] and t.n_padded == g["n_padded"]
    assert t.orig_tokens == g["orig_tokens"]
    N = t.n_tokens
    for key in ("token", "pos", "parent", "subtree_end", "node"):
        assert getattr(t, key)[:N].tolist() == g[key], key
    # pad rows: token 0, pos 0, parent -1, see only themselves
    assert (t.token[N:] == 0).all() and (t.pos[N:] == 0).all()
    assert (t.parent[N:] == -1).all() and (t.node[N:] == -1).all()
    assert t.subtree_end[N:].tolist() == list(range(N, t.n_padded))
    assert (t.root.start_idx, t.root.end_idx) == (-1, -1)
    assert t.root.sequence_ids == g["root"]["sequence_ids"]
    assert t.root.children == {int(k): v for k, v in g["root"]["children"].items()}
    _check_nodes(t, g["nodes"])
    assert {str(k): v.tolist() for k, v in t.seq_index.items()} == g["seq_index"]
    assert t.out_offsets.tolist() == g["out_offsets"]
    M = oracle.dense_mask(t)
    assert [np.nonzero(M[i])[0].tolist() for i in range(N)] == g["visible"]
    assert t.n_pairs == g["n_pairs"] == int(M[:N, :N].sum())
    assert sum(len(s) * (len(s) + 1) // 2 for s in g["seqs"]) == g["causal_pairs"]
    assert t.child_ptr.tolist() == g["child_ptr"]
    assert t.child_idx.tolist() == g["child_idx"]
    for key in ("q_ptr", "q_kb", "q_full", "kb_qhi"):
        assert getattr(t, key).tolist() == g[key], key
    st = oracle.forest_stats(f, g["seqs"])
    assert st["tree_token_ratio"] == pytest.approx(8 / 11)


def test_worked_example_edge():
    g = _load("worked_example_edge.json")
    f = oracle.build_forest(g["seqs"], g["max_tokens_per_mb"])
    t = f.trees[0]
    N = t.n_tokens
    assert N == g["n_tokens"] and t.orig_tokens == g["orig_tokens"]
    for key in ("token", "pos", "parent", "subtree_end", "node"):
        assert getattr(t, key)[:N].tolist() == g[key], key
    _check_nodes(t, g["nodes"])
    assert {str(k): v.tolist() for k, v in t.seq_index.items()} == g["seq_index"]
    assert t.out_offsets.tolist() == g["out_offsets"]


def _ffd_seqs(case):
    seqs = [np.array([1000 * k + p for p in range(L)], dtype=np.int32)
            for k, L in enumerate(case["lengths"])]
    for dst, src, n in case["share"]:
        seqs[dst][:n] = seqs[src][:n]
    return seqs


@pytest.mark.parametrize("case", _load("ffd_cases.json")["cases"], ids=lambda c: c["name"])
def test_ffd_cases(case):
    seqs = _ffd_seqs(case)
    f = oracle.build_forest(seqs, case["capacity"])
    assert [t.seq_ids for t in f.trees] == case["trees"]
    assert [t.n_tokens for t in f.trees] == case["tree_tokens"]
    if "first_token_of_tree0" in case:
        assert int(f.trees[0].token[0]) == case["first_token_of_tree0"]


@pytest.mark.parametrize("seqs,cap,err", [
    ([[1, 2]], 100, oracle.BlockError),
    ([[1, 2]], 0, oracle.InvalidInput),
    ([[1, 2]], -128, oracle.InvalidInput),
    ([], 128, oracle.InvalidInput),
    ([[1], []], 128, oracle.InvalidInput),
    ([list(range(129))], 128, oracle.CapacityError),
])
def test_invalid_inputs(seqs, cap, err):
    with pytest.raises(err):
        oracle.build_forest(seqs, cap)


def test_sequence_of_exactly_capacity():
    f = oracle.build_forest([list(range(1, 129)), list(range(1, 129))], 128)
    assert len(f.trees) == 1 and f.trees[0].n_tokens == 128 and f.trees[0].n_padded == 128


def _random_case(rng):
    """Tiny random sequence sets with lots of accidental sharing."""
    vocab = int(rng.integers(2, 5))
    n = int(rng.integers(1, 7))
    seqs = [rng.integers(0, vocab, size=int(rng.integers(1, 7))).astype(np.int32)
            for _ in range(n)]
    return seqs


def _scaled(rng):
    """Moderate cases spanning several 128-blocks: a few prompt groups."""
    seqs = []
    for _p in range(int(rng.integers(1, 4))):
        prompt = rng.integers(0, 3, size=int(rng.integers(1, 150)))
        for _r in range(int(rng.integers(1, 5))):
            resp = rng.integers(0, 3, size=int(rng.integers(1, 200)))
            seqs.append(np.concatenate([prompt, resp]).astype(np.int32))
    return seqs


def _check_invariants(seqs, cap, f, pad_to_maximum=False):
    seen = []
    for t in f.trees:
        N, Np = t.n_tokens, t.n_padded
        assert N <= cap and Np % BLOCK == 0 and Np <= cap
        assert Np == cap if pad_to_maximum else Np - N < BLOCK
        seen += t.seq_ids
        # packed tokens <-> distinct non-empty prefixes of the tree's sequences
        prefixes = {}
        for sid in t.seq_ids:
            s = [int(x) for x in seqs[sid]]
            idx = t.seq_index[sid]
            assert len(idx) == len(s)
            for p in range(len(s)):
                key = tuple(s[:p + 1])
                assert prefixes.setdefault(key, int(idx[p])) == int(idx[p])
                assert t.token[idx[p]] == s[p] and t.pos[idx[p]] == p
                assert t.parent[idx[p]] == (idx[p - 1] if p else -1)
        assert len(prefixes) == N
        assert sorted(prefixes.values()) == list(range(N))
        # ancestor relation == "prefix of"
        by_flat = {v: k for k, v in prefixes.items()}
        M = oracle.dense_mask(t)
        for i in range(N):
            for j in range(N):
                a, b = by_flat[i], by_flat[j]
                assert M[i, j] == (len(b) <= len(a) and a[:len(b)] == b)
        for i in range(N, Np):
            assert M[i].sum() == 1 and M[i, i]
            assert not M[:N, i].any()
        # subtree_end is the largest query that sees the key
        for j in range(Np):
            assert t.subtree_end[j] == np.nonzero(M[:, j])[0].max()
        # tile classes from a scan of the dense mask
        nb = Np // BLOCK
        exp_ptr, exp_kb, exp_full, exp_cls = [0], [], [], []
        for qb in range(nb):
            for kb in range(nb - 1, -1, -1):
                blk = M[qb * BLOCK:(qb + 1) * BLOCK, kb * BLOCK:(kb + 1) * BLOCK]
                if blk.any():
                    exp_kb.append(kb)
                    exp_full.append(int(blk.all()))
                    bits = 0
                    for qs in range(4):
                        for ks in range(4):
                            sub = blk[32 * qs:32 * qs + 32, 32 * ks:32 * ks + 32]
                            bits |= (0 if not sub.any() else 2 if sub.all() else 1) << (2 * (4 * qs + ks))
                    exp_cls.append(bits)
            exp_ptr.append(len(exp_kb))
        assert t.q_ptr.tolist() == exp_ptr
        assert t.q_kb.tolist() == exp_kb and t.q_full.tolist() == exp_full
        assert t.q_cls.view(np.uint32).tolist() == exp_cls
        assert t.n_pairs == int(M[:N, :N].sum()) == int((t.pos[:N] + 1).sum())
        # child targets: every real token's distinct next tokens
        for i in range(N):
            kids = [c for c in range(N) if t.parent[c] == i]
            assert t.child_idx[t.child_ptr[i]:t.child_ptr[i + 1]].tolist() == kids
        # node table: nodes tile the real tokens, each node's sequences pass
        # through all of its tokens, every sequence is a union of whole nodes
        covered = []
        for k, n in enumerate(t.nodes):
            covered += list(range(n.start_idx, n.end_idx + 1))
            assert (t.node[n.start_idx:n.end_idx + 1] == k).all()
            assert [int(x) for x in t.token[n.start_idx:n.end_idx + 1]] == n.tokens
        assert covered == list(range(N))
        for sid in t.seq_ids:
            idx = set(t.seq_index[sid].tolist())
            for k, n in enumerate(t.nodes):
                span = set(range(n.start_idx, n.end_idx + 1))
                assert span <= idx or not (span & idx)
                assert (sid in n.sequence_ids) == bool(span & idx)
    assert sorted(seen) == list(range(len(seqs)))


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    for _ in range(400):
        seqs = _random_case(rng)
        cap = 128
        f = oracle.build_forest(seqs, cap)
        _check_invariants(seqs, cap, f)


def test_brute_force_tiny_tight_capacity():
    """Scale tiny cases so that the capacity forces several trees."""
    rng = np.random.default_rng(1)
    for _ in range(60):
        base = _random_case(rng)
        seqs = [np.repeat(s, 25) for s in base]       # lengths 25..150
        seqs = [s for s in seqs if len(s) <= 128] or [np.ones(5, np.int32)]
        f = oracle.build_forest(seqs, 128)
        _check_invariants(seqs, 128, f)


def test_brute_force_several_blocks():
    rng = np.random.default_rng(2)
    for _ in range(6):
        seqs = _scaled(rng)
        cap = int(rng.choice([384, 512, 1024]))
        seqs = [s[:cap] for s in seqs]
        f = oracle.build_forest(seqs, cap)
        _check_invariants(seqs, cap, f)


def test_pad_to_maximum():
    """Every tree padded to the capacity: the real part is the default
    build's, pad rows see only themselves (brute force over the dense mask),
    and attention of the real rows does not change."""
    rng = np.random.default_rng(9)
    for it in range(8):
        seqs = _scaled(rng) if it % 2 else _random_case(rng)
        cap = int(rng.choice([256, 384, 512]))
        seqs = [s[:cap] for s in seqs]
        f = oracle.build_forest(seqs, cap, pad_to_maximum=True)
        _check_invariants(seqs, cap, f, pad_to_maximum=True)
        g = oracle.build_forest(seqs, cap)
        assert len(f.trees) == len(g.trees)
        for a, b in zip(f.trees, g.trees):
            N = b.n_tokens
            for name in ("token", "pos", "parent", "subtree_end", "node"):
                assert (getattr(a, name)[:N] == getattr(b, name)[:N]).all(), name
            assert (a.child_ptr == b.child_ptr).all() and (a.child_idx == b.child_idx).all()
            assert all((a.seq_index[s] == b.seq_index[s]).all() for s in b.seq_ids)
            assert a.n_pairs == b.n_pairs
            q = rng.normal(size=(a.n_padded, 2, 8))
            k = rng.normal(size=(a.n_padded, 1, 8))
            v = rng.normal(size=(a.n_padded, 1, 8))
            oa, la = oracle.attn_fwd(a, q, k, v)
            ob, lb = oracle.attn_fwd(b, q[:b.n_padded], k[:b.n_padded], v[:b.n_padded])
            assert np.allclose(oa[:N], ob[:N], rtol=0, atol=1e-12)
