"""The allocation-free backward entry point (pst_tree_attn_bwd_noalloc)
against the workspace one (pst_tree_attn_bwd), through the C ABI: two calls
in a row, the second on a smaller forest, each bitwise equal to the
workspace entry point on the same inputs (the same deterministic kernels;
only where the per-row sums live differs).  Run on its own and after the
other GPU tests: the scratch keeps the last call's contents and must never
leak them into a result."""

import numpy as np
import pytest

from _helpers import Case, attn_inputs, prompt_groups

pytestmark = pytest.mark.gpu


def _one(gpu_lib, seqs, cap, hq, hkv, seed):
    import torch
    case = Case(seqs, cap)
    fmeta = None
    try:
        fmeta = gpu_lib.forest_meta_create(case.forest)
        Np = fmeta.n_padded
        print(f"noalloc case: Np={Np} hq={hq} hkv={hkv}", flush=True)
        q, k, v, do = attn_inputs(Np, hq, hkv, 128, "bf16", seed, with_dout=True)
        o, lse = gpu_lib.tree_attn_fwd(q, k, v, fmeta)
        ref = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, fmeta)
        got = tuple(torch.full_like(x, float("nan")) for x in ref)
        gpu_lib.tree_attn_bwd_noalloc(q, k, v, o, lse, do, fmeta, *got)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        return Np
    finally:
        if fmeta is not None:
            import torch
            torch.cuda.synchronize()
            fmeta.destroy()
        case.close()


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    rng = np.random.default_rng(123)
    big = prompt_groups(rng, 4, 300, 4, 50, 700)
    small = prompt_groups(rng, 1, 100, 2, 10, 60)
    n1 = _one(gpu_lib, big, 2048, 40, 8, 7)      # units plus blocks (5 heads per group)
    n2 = _one(gpu_lib, small, 256, 8, 2, 8)      # units only, a smaller scratch footprint
    assert n2 < n1
