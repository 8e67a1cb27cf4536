"""Gather backward on the GPU against the oracle (through the C ABI).

Tolerance: the kernel forms each element in float32 and rounds it once to the
output type.  bf16 output: |got - ref| <= 2^-8 |ref| + 1e-5 max|ref of the row|
(one bf16 rounding, plus float32 cancellation in A + B (log p + H) measured
against the row's scale); float32 output: 1e-5 |ref| + 1e-5 max|ref of row|.
"""

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_tensor, tree_tensor_seed, worked_example, worked_example_edge

from _helpers import Case, host, prompt_groups

pytestmark = pytest.mark.gpu


def _check_rows(got, ref, dtype, what):
    rtol = 2.0 ** -8 if dtype == "bf16" else 1e-5
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    err = np.abs(got - ref) - (rtol * np.abs(ref) + 1e-5 * scale)
    bad = np.argwhere(err > 0)
    assert bad.size == 0, f"{what}: {len(bad)} elements out of tolerance, first {bad[:3].tolist()}"


def _grads(gpu_lib, tree, meta, n_pad, vocab, dtype, seed, std=2.0):
    import torch
    logits = make_tensor((n_pad, vocab), dtype, seed, "cuda", std=std)
    n = int(tree.out_offsets[-1])
    g = torch.Generator(device="cpu").manual_seed(seed + 7)
    dlp = torch.randn(n, generator=g, dtype=torch.float32).cuda()
    dh = torch.randn(n, generator=g, dtype=torch.float32).cuda()
    dx = gpu_lib.gather_tree_logprobs_entropy_bwd(logits, meta, dlp, dh)
    return logits, dlp, dh, dx


def _full(gpu_lib, seqs, cap, vocab, dtype, seed):
    case = Case(seqs, cap)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"gather bwd case: dtype={dtype} V={vocab} tree={t} N={tree.n_tokens}", flush=True)
            logits, dlp, dh, dx = _grads(gpu_lib, tree, case.metas[t], tree.n_padded, vocab, dtype,
                                         seed + t)
            ref = oracle.gather_logprobs_entropy_bwd(tree, seqs, host(logits), host(dlp), host(dh))
            _check_rows(host(dx), ref, dtype, f"dlogits tree {t}")
            assert (host(dx)[tree.n_tokens:] == 0).all()
    finally:
        case.close()


def test_gather_bwd_worked_example(gpu_lib):
    _full(gpu_lib, worked_example(), 128, 9, "f32", 1)
    _full(gpu_lib, worked_example_edge(), 128, 64, "bf16", 2)


@pytest.mark.parametrize("vocab,dtype", [(1001, "bf16"), (4099, "f32"), (2048, "bf16")])
def test_gather_bwd_several_trees(gpu_lib, vocab, dtype):
    rng = np.random.default_rng(vocab + 1)
    seqs = prompt_groups(rng, 3, 60, 4, 10, 120, vocab=min(vocab, 500))
    _full(gpu_lib, seqs, 384, vocab, dtype, vocab)


def test_gather_bwd_repeated_targets(gpu_lib):
    """Duplicate sequences and a shared prefix: several outputs of one row
    with the same next token must add up once into that entry."""
    seqs = [np.array([5, 6, 7, 8], np.int32), np.array([5, 6, 7, 8], np.int32),
            np.array([5, 6, 9], np.int32), np.array([5, 6, 7, 1, 2], np.int32)]
    _full(gpu_lib, seqs, 128, 16, "f32", 11)
    _full(gpu_lib, seqs, 128, 16, "bf16", 12)


def test_gather_bwd_grpo_sampled(gpu_lib):
    """Full-size grpo trees (32000-entry rows): every output computed on the
    GPU, sampled rows (branch rows among them) checked against the oracle."""
    w = get_workload("grpo")
    case = Case(w.seqs, w.max_tokens_per_mb)
    rng = np.random.default_rng(2)
    try:
        for t, tree in enumerate(case.ref.trees[:2]):
            print(f"gather bwd sampled: grpo tree={t} N={tree.n_tokens}", flush=True)
            logits, dlp, dh, dx = _grads(gpu_lib, tree, case.metas[t], tree.n_padded, w.vocab,
                                         w.dtype, tree_tensor_seed(w.seed, t, "dlogits"),
                                         std=w.logit_std)
            kids = np.diff(tree.child_ptr[:tree.n_tokens + 1])
            branch = np.nonzero(kids > 1)[0]
            rows = sorted(set(rng.choice(tree.n_tokens, size=10, replace=False).tolist())
                          | set(branch[:6].tolist()) | {tree.n_tokens - 1})
            lg = {r: host(logits[r]) for r in rows}
            ref = oracle.gather_logprobs_entropy_bwd(tree, w.seqs, lg, host(dlp), host(dh), rows=rows)
            got = host(dx)
            for r in rows:
                _check_rows(got[r][None], ref[r][None], w.dtype, f"dlogits row {r}")
            assert (got[tree.n_tokens:] == 0).all()
    finally:
        case.close()


def test_gather_bwd_deterministic(gpu_lib):
    import torch
    rng = np.random.default_rng(4)
    seqs = prompt_groups(rng, 2, 50, 4, 10, 100, vocab=300)
    case = Case(seqs, 256)
    try:
        tree = case.ref.trees[0]
        logits, dlp, dh, a = _grads(gpu_lib, tree, case.metas[0], tree.n_padded, 3001, "bf16", 9)
        b = gpu_lib.gather_tree_logprobs_entropy_bwd(logits, case.metas[0], dlp, dh)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        case.close()


def test_gather_bwd_rejects_misaligned_pair(gpu_lib):
    import torch
    case = Case(worked_example(), 128)
    try:
        n = int(case.ref.trees[0].out_offsets[-1])
        buf = torch.zeros(128 * 9 + 4, dtype=torch.float32, device="cuda")
        logits = buf[:128 * 9].view(128, 9)
        dlogits = torch.zeros(128 * 9 + 1, dtype=torch.float32, device="cuda")[1:].view(128, 9)
        d = torch.zeros(n, dtype=torch.float32, device="cuda")
        with pytest.raises(gpu_lib.PstError) as e:
            gpu_lib.gather_tree_logprobs_entropy_bwd(logits, case.metas[0], d, d, dlogits=dlogits)
        assert e.value.name == "PST_ESHAPE"
    finally:
        case.close()


@pytest.mark.parametrize("vocab,dtype", [(40000, "bf16"), (20011, "f32"), (3001, "bf16")])
def test_gather_bwd_with_forward_row_stats(gpu_lib, vocab, dtype):
    """The forward's saved (lse, entropy) per row: checked against the oracle's
    row statistics, then fed to the backward (rows beyond the register-resident
    size take the one-read path), which must match the oracle as without them."""
    import torch
    rng = np.random.default_rng(vocab)
    seqs = prompt_groups(rng, 3, 40, 3, 10, 90, vocab=500)
    case = Case(seqs, 256)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"gather row stats case: dtype={dtype} V={vocab} tree={t}", flush=True)
            meta = case.metas[t]
            logits = make_tensor((tree.n_padded, vocab), dtype, vocab + t, "cuda", std=2.0)
            stats = torch.zeros((tree.n_padded, 2), dtype=torch.float32, device="cuda")
            gpu_lib.gather_tree_logprobs_entropy(logits, meta, row_stats=stats)
            N = tree.n_tokens
            lse, ent = oracle.row_lse_entropy(host(logits)[:N])
            st = host(stats)
            assert np.abs(st[:N, 0] - lse).max() <= 1e-4 * np.abs(lse).max() + 1e-5
            assert np.abs(st[:N, 1] - ent).max() <= 1e-4 * np.abs(ent).max() + 1e-5
            n = int(tree.out_offsets[-1])
            g = torch.Generator(device="cpu").manual_seed(vocab + 7 + t)
            dlp = torch.randn(n, generator=g, dtype=torch.float32).cuda()
            dh = torch.randn(n, generator=g, dtype=torch.float32).cuda()
            dx = gpu_lib.gather_tree_logprobs_entropy_bwd(logits, meta, dlp, dh, row_stats=stats)
            ref = oracle.gather_logprobs_entropy_bwd(tree, seqs, host(logits), host(dlp), host(dh))
            _check_rows(host(dx), ref, dtype, f"dlogits tree {t} (row stats)")
            assert (host(dx)[N:] == 0).all()
    finally:
        case.close()


def test_gather_bwd_bimodal_sampled_row_stats(gpu_lib):
    """Full-size bimodal trees (152064-entry rows) through the forward with
    row statistics and the one-read backward, sampled rows against the oracle."""
    import torch
    w = get_workload("bimodal")
    case = Case(w.seqs, w.max_tokens_per_mb)
    rng = np.random.default_rng(4)
    try:
        tree = case.ref.trees[0]
        meta = case.metas[0]
        print(f"gather bwd sampled: bimodal tree=0 N={tree.n_tokens}", flush=True)
        logits = make_tensor((tree.n_padded, w.vocab), w.dtype, tree_tensor_seed(w.seed, 0, "logits"),
                             "cuda", std=w.logit_std)
        stats = torch.empty((tree.n_padded, 2), dtype=torch.float32, device="cuda")
        gpu_lib.gather_tree_logprobs_entropy(logits, meta, row_stats=stats)
        n = int(tree.out_offsets[-1])
        g = torch.Generator(device="cpu").manual_seed(99)
        dlp = torch.randn(n, generator=g, dtype=torch.float32).cuda()
        dh = torch.randn(n, generator=g, dtype=torch.float32).cuda()
        dx = gpu_lib.gather_tree_logprobs_entropy_bwd(logits, meta, dlp, dh, row_stats=stats)
        torch.cuda.synchronize()
        kids = np.diff(tree.child_ptr[:tree.n_tokens + 1])
        branch = np.nonzero(kids > 1)[0]
        rows = sorted(set(rng.choice(tree.n_tokens, size=8, replace=False).tolist())
                      | set(branch[:4].tolist()) | {tree.n_tokens - 1})
        lg = {r: host(logits[r]) for r in rows}
        ref = oracle.gather_logprobs_entropy_bwd(tree, w.seqs, lg, host(dlp), host(dh), rows=rows)
        for r in rows:
            _check_rows(host(dx[r])[None], ref[r][None], w.dtype, f"dlogits row {r}")
        assert int((dx[tree.n_tokens:] != 0).sum()) == 0
    finally:
        case.close()

def _degenerate_inputs():
    """Single-token sequences (two identical, one a prefix of longer ones),
    and trees of exactly 128 and of 129 tokens."""
    rng = np.random.default_rng(79)
    singles = [np.array([5], np.int32), np.array([5], np.int32), np.array([9], np.int32),
               np.array([3], np.int32), np.array([3, 4, 5, 6], np.int32), np.array([3, 4], np.int32)]
    return [(singles, 128), ([rng.integers(0, 500, 128).astype(np.int32)], 128),
            ([rng.integers(0, 500, 129).astype(np.int32)], 256)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_bwd_degenerate_inputs(gpu_lib, dtype):
    for i, (seqs, cap) in enumerate(_degenerate_inputs()):
        _full(gpu_lib, seqs, cap, 512, dtype, 80 + i)
