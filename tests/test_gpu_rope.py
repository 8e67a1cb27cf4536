"""Tree-position rotary embedding on the GPU against the oracle (through the
C ABI).

Tolerance: angles are formed in float64 and the rotation in float32, so fp32
results match to 1e-5 |ref| + 1e-6 (positions up to 32767); bf16 results to
one output rounding, 2^-8 |ref| + 1e-6.
"""

import numpy as np
import pytest

import oracle
from workloads import get_workload, make_tensor, worked_example

from _helpers import Case, assert_close, host, prompt_groups

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return dict(rtol=2.0 ** -8, atol=1e-6) if dtype == "bf16" else dict(rtol=1e-5, atol=1e-6)


def _run(gpu_lib, seqs, cap, heads, d, dtype, seed, theta=None, inverse=False):
    case = Case(seqs, cap)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"rope case: dtype={dtype} heads={heads} d={d} tree={t} Np={tree.n_padded}", flush=True)
            x = make_tensor((tree.n_padded, heads, d), dtype, seed + t, "cuda")
            x0 = host(x)
            gpu_lib.tree_rope(x, case.metas[t], theta=theta, inverse=inverse)
            ref = oracle.rope(x0, tree.pos, theta=theta or 10000.0, inverse=inverse)
            ref[tree.n_tokens:] = x0[tree.n_tokens:]   # pad rows untouched
            assert_close(host(x), ref, dtype, "rope", **_tol(dtype))
    finally:
        case.close()


def test_rope_worked_example(gpu_lib):
    _run(gpu_lib, worked_example(), 128, 2, 64, "f32", 1)
    _run(gpu_lib, worked_example(), 128, 4, 128, "bf16", 2, theta=500.0)


@pytest.mark.parametrize("heads,d,dtype", [(32, 128, "bf16"), (8, 128, "f32"), (5, 64, "bf16"),
                                           (3, 16, "bf16"), (2, 8, "f32")])
def test_rope_several_trees(gpu_lib, heads, d, dtype):
    rng = np.random.default_rng(heads * 7 + d)
    seqs = prompt_groups(rng, 3, 150, 3, 20, 260)
    _run(gpu_lib, seqs, 1024, heads, d, dtype, heads + d)


def test_rope_inverse_roundtrip(gpu_lib):
    """The inverse rotation undoes the forward (fp32, to rounding)."""
    import torch
    seqs = worked_example()
    case = Case(seqs, 128)
    try:
        x = make_tensor((128, 4, 64), "f32", 5, "cuda")
        y = x.clone()
        gpu_lib.tree_rope(y, case.metas[0])
        gpu_lib.tree_rope(y, case.metas[0], inverse=True)
        torch.cuda.synchronize()
        assert (y - x).abs().max().item() < 1e-5
    finally:
        case.close()


def test_rope_long_positions(gpu_lib):
    """Depths up to 8192 + 4096 (the long workload's first tree): float64
    angles keep fp32 results at 1e-5."""
    w = get_workload("long")
    case = Case(w.seqs, w.max_tokens_per_mb)
    try:
        tree = case.ref.trees[0]
        x = make_tensor((tree.n_padded, 2, 128), "f32", 9, "cuda")
        x0 = host(x)
        gpu_lib.tree_rope(x, case.metas[0])
        ref = oracle.rope(x0, tree.pos)
        ref[tree.n_tokens:] = x0[tree.n_tokens:]
        assert_close(host(x), ref, "f32", "rope[long]", rtol=1e-5, atol=1e-5)
    finally:
        case.close()


def test_rope_forest_meta_matches_per_tree(gpu_lib):
    import torch
    rng = np.random.default_rng(8)
    seqs = prompt_groups(rng, 4, 100, 3, 10, 200)
    case = Case(seqs, 384)
    try:
        fmeta = gpu_lib.forest_meta_create(case.forest)
        Np = sum(t.n_padded for t in case.ref.trees)
        x = make_tensor((Np, 8, 128), "bf16", 31, "cuda")
        y = x.clone()
        gpu_lib.tree_rope(x, fmeta)
        r0 = 0
        for t, tree in enumerate(case.ref.trees):
            part = y[r0:r0 + tree.n_padded].contiguous()
            gpu_lib.tree_rope(part, case.metas[t])
            torch.cuda.synchronize()
            assert torch.equal(x[r0:r0 + tree.n_padded], part)
            r0 += tree.n_padded
        torch.cuda.synchronize()
        fmeta.destroy()
    finally:
        case.close()


def test_rope_rejects_bad_head_dim(gpu_lib):
    case = Case(worked_example(), 128)
    try:
        x = make_tensor((128, 2, 24), "bf16", 1, "cuda")
        with pytest.raises(gpu_lib.PstError) as e:
            gpu_lib.tree_rope(x, case.metas[0])
        assert e.value.name == "PST_ESHAPE"
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
def test_rope_degenerate_inputs(gpu_lib, dtype):
    for i, (seqs, cap) in enumerate(_degenerate_inputs()):
        _run(gpu_lib, seqs, cap, 8, 128, dtype, 70 + i)
