"""The library's host builder (C++ behind the C ABI) against the oracle:
every integer array bit-exact, on the worked example, hand-worked packing
cases, brute-force tiny sequence sets and all synthetic workloads (CPU only;
the builder never touches the GPU)."""

import json
import os

import numpy as np
import pytest

import oracle
import prefix_shared_tree_packed_amd as pst
from workloads import WORKLOADS, get_workload, worked_example, worked_example_edge

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def compare_forest(seqs, cap, pad_to_maximum=False):
    ref = oracle.build_forest(seqs, cap, pad_to_maximum=pad_to_maximum)
    got = pst.build_tree(seqs, cap, pad_to_maximum=pad_to_maximum)
    assert got.n_trees == len(ref.trees)
    assert got.seq_tree().tolist() == ref.seq_tree.tolist()
    for t, rt in enumerate(ref.trees):
        e = got.export(t)
        s = got.sizes(t)
        assert s["n_tokens"] == rt.n_tokens and s["n_padded"] == rt.n_padded
        assert s["n_pairs"] == rt.n_pairs
        for key in ("token", "pos", "parent", "subtree_end", "node", "child_ptr", "child_idx",
                    "q_ptr", "q_kb", "q_full", "q_cls", "kb_qhi", "fwd_order", "bwd_order"):
            np.testing.assert_array_equal(e[key], getattr(rt, key), err_msg=key)
        assert e["seq_ids"].tolist() == rt.seq_ids
        assert e["seq_out_offsets"].tolist() == rt.out_offsets.tolist()
        np.testing.assert_array_equal(
            e["seq_index"], np.concatenate([rt.seq_index[s] for s in rt.seq_ids]))
        assert e["node_start"].tolist() == [n.start_idx for n in rt.nodes]
        assert e["node_end"].tolist() == [n.end_idx for n in rt.nodes]
        assert e["node_parent"].tolist() == [n.parent for n in rt.nodes]
        ptr, ids = e["node_seq_ptr"], e["node_seq_ids"]
        assert [ids[ptr[k]:ptr[k + 1]].tolist() for k in range(len(rt.nodes))] == \
            [n.sequence_ids for n in rt.nodes]
    st, rst = got.stats(), oracle.forest_stats(ref, seqs)
    for key in ("n_trees", "tree_tokens", "padded_tokens", "orig_tokens", "n_tiles"):
        assert st[key] == rst[key], key
    assert st["n_pairs"] == rst["pairs"] and st["causal_pairs"] == rst["causal_pairs"]
    assert st["tree_token_ratio"] == pytest.approx(rst["tree_token_ratio"], rel=1e-15)
    return got, ref


def test_worked_examples():
    compare_forest(worked_example(), 128)
    compare_forest(worked_example_edge(), 128)


def test_ffd_cases():
    with open(os.path.join(GOLD, "ffd_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        seqs = [np.array([1000 * k + p for p in range(L)], dtype=np.int32)
                for k, L in enumerate(case["lengths"])]
        for dst, src, n in case["share"]:
            seqs[dst][:n] = seqs[src][:n]
        got, _ = compare_forest(seqs, case["capacity"])
        assert [got.export(t)["seq_ids"].tolist() for t in range(got.n_trees)] == case["trees"]


def test_brute_force_random():
    rng = np.random.default_rng(11)
    for trial in range(300):
        vocab = int(rng.integers(2, 5))
        n = int(rng.integers(1, 8))
        scale = 1 if trial % 3 else 30
        seqs = [np.repeat(rng.integers(0, vocab, size=int(rng.integers(1, 7))), scale).astype(np.int32)
                for _ in range(n)]
        cap = int(rng.choice([128, 256])) if scale > 1 else 128
        seqs = [s[:cap] for s in seqs]
        compare_forest(seqs, cap)


def test_pad_to_maximum():
    rng = np.random.default_rng(12)
    for trial in range(40):
        n = int(rng.integers(1, 8))
        seqs = [np.repeat(rng.integers(0, 4, size=int(rng.integers(1, 7))), 30).astype(np.int32)
                for _ in range(n)]
        cap = int(rng.choice([128, 256, 384]))
        compare_forest([s[:cap] for s in seqs], cap, pad_to_maximum=True)
    w = get_workload("grpo")
    compare_forest(w.seqs, w.max_tokens_per_mb, pad_to_maximum=True)


def test_wide_nodes():
    """A root with many children (the builder indexes wide nodes by hash)."""
    rng = np.random.default_rng(3)
    seqs = [np.array([t] + list(rng.integers(0, 3, size=5)), np.int32) for t in rng.permutation(60)]
    seqs += [np.array([7, 1, 2], np.int32), np.array([7, 1, 2, 9], np.int32)]
    compare_forest(seqs, 1024)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workloads(name):
    w = get_workload(name)
    compare_forest(w.seqs, w.max_tokens_per_mb)


@pytest.mark.parametrize("seqs,cap,code", [
    ([[1, 2]], 100, "PST_EBLOCK"),
    ([[1, 2]], 0, "PST_EINVAL"),
    ([[1, 2]], -128, "PST_EINVAL"),
    ([], 128, "PST_EINVAL"),
    ([[1], []], 128, "PST_EINVAL"),
    ([list(range(129))], 128, "PST_ECAPACITY"),
])
def test_errors_match_oracle(seqs, cap, code):
    with pytest.raises(oracle.OracleError) as oe:
        oracle.build_forest(seqs, cap)
    with pytest.raises(pst.PstError) as pe:
        pst.build_tree(seqs, cap)
    assert pe.value.name == code == "PST_" + oe.value.code
