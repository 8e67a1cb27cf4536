"""Logprob/entropy gather on the GPU against the oracle (through the C ABI)."""

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_tensor, tree_tensor_seed, worked_example, worked_example_edge

from _helpers import Case, assert_close, host, prompt_groups

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return dict(rtol=0.0, atol=1e-3) if dtype == "bf16" else dict(rtol=1e-5, atol=1e-6)


def _run(gpu_lib, seqs, cap, vocab, dtype, seed, std=1.0, seq_sample=None):
    case = Case(seqs, cap)
    rng = np.random.default_rng(seed)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"gather case: dtype={dtype} V={vocab} tree={t} N={tree.n_tokens}", flush=True)
            logits = make_tensor((tree.n_padded, vocab), dtype, tree_tensor_seed(seed, t, "logits"),
                                 "cuda", std=std)
            lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, case.metas[t])
            lph, enth = host(lp), host(ent)
            ids = tree.seq_ids
            if seq_sample is not None and len(ids) > seq_sample:
                ids = sorted(rng.choice(ids, size=seq_sample, replace=False).tolist())
            lg = host(logits[:tree.n_tokens])
            for sid in ids:
                k = tree.seq_ids.index(sid)
                a, b = tree.out_offsets[k], tree.out_offsets[k + 1]
                sub = oracle.Tree(**{**tree.__dict__, "seq_ids": [sid],
                                     "out_offsets": np.array([0, b - a])})
                rlp, rent = oracle.gather_logprobs_entropy(sub, seqs, lg)
                assert_close(lph[a:b], rlp, dtype, f"logprob seq {sid}", **_tol(dtype))
                assert_close(enth[a:b], rent, dtype, f"entropy seq {sid}", **_tol(dtype))
    finally:
        case.close()


def test_gather_worked_example(gpu_lib):
    _run(gpu_lib, worked_example(), 128, 9, "f32", 1)       # 36-byte rows: unaligned
    _run(gpu_lib, worked_example_edge(), 128, 64, "bf16", 2, std=2.0)


def test_gather_tiny_workload(gpu_lib):
    w = get_workload("tiny")
    _run(gpu_lib, w.seqs, w.max_tokens_per_mb, w.vocab, w.dtype, w.seed, std=w.logit_std)


@pytest.mark.parametrize("vocab,dtype", [(1001, "bf16"), (4099, "f32"), (32000, "bf16")])
def test_gather_several_trees(gpu_lib, vocab, dtype):
    rng = np.random.default_rng(vocab)
    seqs = prompt_groups(rng, 4, 100, 4, 10, 200, vocab=min(vocab, 1000))
    _run(gpu_lib, seqs, 512, vocab, dtype, vocab, std=2.0)


def test_gather_closed_forms(gpu_lib):
    """Uniform logits: logprob = -log V, entropy = log V (0 on last tokens)."""
    import torch
    seqs = worked_example_edge()
    case = Case(seqs, 128)
    try:
        V = 32000
        logits = torch.full((128, V), 0.5, dtype=torch.bfloat16, device="cuda")
        lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, case.metas[0])
        lph, enth = host(lp), host(ent)
        last = set((case.ref.trees[0].out_offsets[1:] - 1).tolist())
        for p in range(len(lph)):
            assert abs(lph[p] - (0.0 if p in last else -np.log(V))) < 1e-3
            assert abs(enth[p] - np.log(V)) < 1e-3
    finally:
        case.close()


def test_gather_grpo_full(gpu_lib):
    w = get_workload("grpo")
    _run(gpu_lib, w.seqs, w.max_tokens_per_mb, w.vocab, w.dtype, w.seed, std=w.logit_std)


def test_gather_bimodal_sampled(gpu_lib):
    w = get_workload("bimodal")
    seqs = w.seqs
    case_trees = oracle.build_forest(seqs, w.max_tokens_per_mb).trees
    # keep three trees' sequences only: the gather is per tree
    keep = set(case_trees[0].seq_ids) | set(case_trees[5].seq_ids) | set(case_trees[-1].seq_ids)
    sub = [s for i, s in enumerate(seqs) if i in keep]
    _run(gpu_lib, sub, w.max_tokens_per_mb, w.vocab, w.dtype, w.seed, std=w.logit_std, seq_sample=4)


def test_gather_rejects_out_of_vocab(gpu_lib):
    import torch
    case = Case(worked_example(), 128)
    try:
        logits = torch.zeros((128, 8), dtype=torch.float32, device="cuda")  # token 8 needs V > 8
        with pytest.raises(gpu_lib.PstError) as e:
            gpu_lib.gather_tree_logprobs_entropy(logits, case.metas[0])
        assert e.value.name == "PST_EINVAL"
    finally:
        case.close()


def test_gather_forest_meta_matches_per_tree(gpu_lib):
    import torch
    rng = np.random.default_rng(8)
    seqs = prompt_groups(rng, 5, 120, 3, 10, 200, vocab=1000)
    case = Case(seqs, 384)
    try:
        fmeta = gpu_lib.forest_meta_create(case.forest)
        Np = sum(t.n_padded for t in case.ref.trees)
        logits = make_tensor((Np, 1001), "bf16", 77, "cuda", std=2.0)
        lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, fmeta)
        r0, o0 = 0, 0
        for t, tree in enumerate(case.ref.trees):
            lpt, entt = gpu_lib.gather_tree_logprobs_entropy(
                logits[r0:r0 + tree.n_padded].contiguous(), case.metas[t])
            n = int(tree.out_offsets[-1])
            torch.cuda.synchronize()
            assert torch.equal(lp[o0:o0 + n], lpt) and torch.equal(ent[o0:o0 + n], entt)
            r0 += tree.n_padded
            o0 += n
        assert o0 == lp.numel()
        torch.cuda.synchronize()
        fmeta.destroy()
    finally:
        case.close()


def test_gather_masked_vocabulary(gpu_lib):
    """Rows whose vocabulary is partly masked to -inf (odd vocabulary, so
    rows are unaligned and also take the element-wise head/tail path):
    finite entropy and logprobs equal to the oracle's, where 0 log 0 = 0."""
    import torch
    rng = np.random.default_rng(17)
    seqs = prompt_groups(rng, 2, 40, 3, 10, 60, vocab=300)
    case = Case(seqs, 256)
    try:
        for dtype in ("bf16", "f32"):
            for t, tree in enumerate(case.ref.trees):
                logits = make_tensor((tree.n_padded, 1003), dtype, 1000 + t, "cuda", std=2.0)
                logits[:, 300:] = float("-inf")   # every target (< 300) stays visible
                lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, case.metas[t])
                lph, enth = host(lp), host(ent)
                assert np.isfinite(enth).all() and np.isfinite(lph).all()
                lg = host(logits[:tree.n_tokens])
                rlp, rent = oracle.gather_logprobs_entropy(tree, seqs, lg)
                assert_close(lph, rlp, dtype, "logprob[masked]", **_tol(dtype))
                assert_close(enth, rent, dtype, "entropy[masked]", **_tol(dtype))
    finally:
        case.close()

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_degenerate_inputs(gpu_lib, dtype):
    """Single-token sequences (logprob 0 at the only position; two identical
    ones and one that is a prefix of longer sequences), and trees of exactly
    128 and 129 tokens."""
    rng = np.random.default_rng(78)
    singles = [np.array([5], np.int32), np.array([5], np.int32), np.array([9], np.int32),
               np.array([3], np.int32), np.array([3, 4, 5, 6], np.int32), np.array([3, 4], np.int32)]
    _run(gpu_lib, singles, 128, 64, dtype, 11)
    _run(gpu_lib, [rng.integers(0, 500, 128).astype(np.int32)], 128, 512, dtype, 12)
    _run(gpu_lib, [rng.integers(0, 500, 129).astype(np.int32)], 256, 512, dtype, 13)
