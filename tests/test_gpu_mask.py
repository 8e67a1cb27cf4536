"""Dense mask export and pad_to_maximum trees on the GPU against the oracle
(through the C ABI).

The exported mask is compared bit for bit with the oracle's dense ancestor
mask (parent-chain walks): every element on small cases and on a forest's
block-diagonal mask, sampled rows plus the visible count on a full-size
8192-row tree.  Trees padded to the capacity go through attention forward
and backward, the gather and RoPE, compared as elsewhere."""

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_tensor, tree_tensor_seed, worked_example

from _helpers import Case, assert_close, attn_inputs, host, host32, prompt_groups

pytestmark = pytest.mark.gpu

FORMATS = ("u8", "add_f32", "add_bf16")


def _expected(M, fmt):
    if fmt == "u8":
        return M.astype(np.float64)
    return np.where(M, 0.0, -np.inf)


def _check_mask(got, M, fmt, what):
    g = host(got)
    exp = _expected(M, fmt)
    bad = np.argwhere(g != exp)
    assert bad.size == 0, f"{what} [{fmt}]: {len(bad)} wrong elements, first {bad[:4].tolist()}"


@pytest.mark.parametrize("fmt", FORMATS)
def test_mask_small(gpu_lib, fmt):
    rng = np.random.default_rng(5)
    for seqs, cap in ((worked_example(), 128), (prompt_groups(rng, 3, 150, 3, 20, 260), 1024),
                      (prompt_groups(rng, 4, 40, 4, 10, 90), 256)):
        case = Case(seqs, cap)
        try:
            for t, tree in enumerate(case.ref.trees):
                print(f"mask case: fmt={fmt} cap={cap} tree={t} Np={tree.n_padded}", flush=True)
                got = gpu_lib.tree_dense_mask(case.metas[t], fmt)
                _check_mask(got, oracle.dense_mask(tree), fmt, f"tree {t}")
        finally:
            case.close()


def test_mask_forest_block_diagonal(gpu_lib):
    import torch
    rng = np.random.default_rng(6)
    seqs = prompt_groups(rng, 4, 60, 4, 20, 120)
    case = Case(seqs, 384)
    try:
        assert len(case.ref.trees) > 1
        meta = gpu_lib.forest_meta_create(case.forest)
        print(f"mask case: forest of {len(case.ref.trees)} trees, Np={meta.n_padded}", flush=True)
        got = gpu_lib.tree_dense_mask(meta, "u8")
        torch.cuda.synchronize()
        M = np.zeros((meta.n_padded, meta.n_padded), dtype=bool)
        off = 0
        for tree in case.ref.trees:
            M[off:off + tree.n_padded, off:off + tree.n_padded] = oracle.dense_mask(tree)
            off += tree.n_padded
        _check_mask(got, M, "u8", "forest")
        meta.destroy()
    finally:
        case.close()


def test_mask_grpo_full_size_sampled(gpu_lib):
    import torch
    w = get_workload("grpo")
    case = Case(w.seqs, w.max_tokens_per_mb)
    try:
        tree = case.ref.trees[0]
        print(f"mask case: grpo tree 0, Np={tree.n_padded}", flush=True)
        got = gpu_lib.tree_dense_mask(case.metas[0], "u8")
        torch.cuda.synchronize()
        n_pad = tree.n_padded - tree.n_tokens
        assert int(got.sum(dtype=torch.int64)) == tree.n_pairs + n_pad
        rng = np.random.default_rng(7)
        rows = np.unique(np.concatenate([rng.integers(0, tree.n_padded, 48),
                                         [0, tree.n_tokens - 1, tree.n_padded - 1]]))
        sub = got[torch.as_tensor(rows, device=got.device)].cpu().numpy()
        for r, row in zip(rows, sub):
            exp = np.zeros(tree.n_padded, dtype=np.uint8)
            exp[oracle.ancestors(tree, int(r))] = 1
            assert (row == exp).all(), f"row {r}"
    finally:
        case.close()


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 8, 2, 128)])
def test_pad_to_maximum_path(gpu_lib, dtype, hq, hkv, d):
    """Trees padded to the capacity (several pad-only blocks) through every
    device entry point."""
    rng = np.random.default_rng(hq + d)
    seqs = prompt_groups(rng, 2, 100, 3, 20, 200)
    case = Case(seqs, 1024, pad_to_maximum=True)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"pad_to_maximum case: dtype={dtype} tree={t} N={tree.n_tokens} "
                  f"Np={tree.n_padded}", flush=True)
            assert tree.n_padded == 1024 and case.metas[t].n_padded == 1024
            q, k, v, do = attn_inputs(tree.n_padded, hq, hkv, d, dtype, 70 + t, with_dout=True)
            _check_mask(gpu_lib.tree_dense_mask(case.metas[t], "u8"), oracle.dense_mask(tree),
                        "u8", "pad_to_maximum mask")
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, case.metas[t])
            O, LSE = oracle.attn_fwd(tree, host(q), host(k), host(v))
            assert_close(host(o), O, dtype, "O")
            assert_close(host(lse), LSE, dtype, "LSE")
            dq, dk, dv = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, case.metas[t])
            args = (tree, host(q), host(k), host(v), host(do))
            rdq, rdk, rdv = oracle.attn_bwd(*args)
            mdq, mdk, mdv = oracle.attn_bwd_magnitudes(*args) if dtype == "f32" else (None,) * 3
            assert_close(host(dq), rdq, dtype, "dQ", grad=True, mag=mdq)
            assert_close(host(dk), rdk, dtype, "dK", grad=True, mag=mdk)
            assert_close(host(dv), rdv, dtype, "dV", grad=True, mag=mdv)
            qr = q.clone()
            gpu_lib.tree_rope(qr, case.metas[t])
            ref = oracle.rope(host(q), tree.pos)
            assert_close(host(qr), ref, dtype, "rope", rtol=2.0 ** -8 if dtype == "bf16" else 1e-5,
                         atol=1e-6)
            vocab = 1024  # token ids are drawn below 1000
            logits = make_tensor((tree.n_padded, vocab), dtype, tree_tensor_seed(80, t, "logits"),
                                 "cuda", std=2.0)
            lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, case.metas[t])
            rlp, rent = oracle.gather_logprobs_entropy(tree, seqs, host32(logits))
            tol = 1e-3 if dtype == "bf16" else None
            assert_close(host(lp), rlp, "f32", "logprobs", rtol=0 if tol else None, atol=tol)
            assert_close(host(ent), rent, "f32", "entropy", rtol=0 if tol else None, atol=tol)
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


@pytest.mark.parametrize("fmt", FORMATS)
def test_mask_degenerate_inputs(gpu_lib, fmt):
    for seqs, cap in _degenerate_inputs():
        case = Case(seqs, cap)
        try:
            for t, tree in enumerate(case.ref.trees):
                M = oracle.dense_mask(tree)
                got = gpu_lib.tree_dense_mask(case.metas[t], fmt)
                _check_mask(got, M, fmt, f"tree {t} ({len(seqs)} sequences, cap {cap})")
        finally:
            case.close()
