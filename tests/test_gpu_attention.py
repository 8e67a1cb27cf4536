"""Tree attention forward/backward on the GPU against the oracle (through the
C ABI).  Small cases are compared element by element over every output;
full-size workloads on sampled rows that the oracle evaluates one by one."""

import numpy as np
import pytest

import oracle
from workloads import get_workload, worked_example, worked_example_edge

from _helpers import Case, assert_close, attn_inputs, host, host32, prompt_groups

pytestmark = pytest.mark.gpu


def _fwd_full(gpu_lib, seqs, cap, hq, hkv, d, dtype, seed, scale=None):
    case = Case(seqs, cap)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"fwd case: dtype={dtype} hq={hq} hkv={hkv} d={d} tree={t} Np={tree.n_padded}", flush=True)
            q, k, v = attn_inputs(tree.n_padded, hq, hkv, d, dtype, seed + t)
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, case.metas[t], softmax_scale=scale)
            O, LSE = oracle.attn_fwd(tree, host(q), host(k), host(v), scale=scale)
            assert_close(host(o), O, dtype, "O")
            assert_close(host(lse), LSE, dtype, "LSE")
    finally:
        case.close()


def test_fwd_worked_example_fp32(gpu_lib):
    _fwd_full(gpu_lib, worked_example(), 128, 2, 1, 64, "f32", 1)
    _fwd_full(gpu_lib, worked_example_edge(), 128, 2, 2, 64, "f32", 2)


def test_fwd_worked_example_bf16(gpu_lib):
    # 4 and 5 query heads per key/value head: units of four heads, and units
    # plus 128-query blocks for the fifth, on a single 128-row tree
    _fwd_full(gpu_lib, worked_example(), 128, 4, 1, 128, "bf16", 3)
    _fwd_full(gpu_lib, worked_example(), 128, 5, 1, 128, "bf16", 5)
    _fwd_full(gpu_lib, worked_example(), 128, 2, 2, 64, "bf16", 4, scale=0.2)


def test_fwd_tiny_workload(gpu_lib):
    w = get_workload("tiny")
    _fwd_full(gpu_lib, w.seqs, w.max_tokens_per_mb, w.hq, w.hkv, w.head_dim, w.dtype, w.seed)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 8, 2, 128),
                                             ("bf16", 5, 1, 64), ("bf16", 6, 6, 128),
                                             ("bf16", 10, 2, 128), ("bf16", 12, 2, 128),
                                             ("bf16", 16, 2, 128), ("bf16", 6, 2, 128),
                                             ("bf16", 20, 2, 128)])
def test_fwd_several_tiles(gpu_lib, dtype, hq, hkv, d):
    """Trees spanning several 128-blocks with a ragged tail, several trees.
    bf16 head_dim 128 with 4, 5, 6, 8 or 10 query heads per key/value head
    runs 32-query units of four heads (two per group at 8 and 10, with
    128-query blocks for the rest at 5, 6 and 10); 1 or 3 per group runs
    128-query blocks only."""
    rng = np.random.default_rng(hq * 7 + d)
    seqs = prompt_groups(rng, 3, 150, 3, 20, 260)
    _fwd_full(gpu_lib, seqs, 1024, hq, hkv, d, dtype, 10 + hq)


def test_fwd_no_sharing(gpu_lib):
    """Distinct sequences: every tree token sees exactly its causal prefix."""
    rng = np.random.default_rng(5)
    seqs = [np.concatenate([[i], rng.integers(0, 50, size=int(rng.integers(100, 400)))]).astype(np.int32)
            for i in range(5)]
    _fwd_full(gpu_lib, seqs, 1024, 8, 2, 128, "bf16", 21)


def test_fwd_single_long_chain(gpu_lib):
    """One sequence filling its tree exactly: plain causal attention, every
    off-diagonal tile full."""
    seqs = [np.arange(1, 641, dtype=np.int32)]
    _fwd_full(gpu_lib, seqs, 640, 4, 4, 64, "f32", 22)
    _fwd_full(gpu_lib, seqs, 640, 8, 2, 128, "bf16", 23)


def _fwd_sampled(gpu_lib, name, n_rows=48, n_trees=None):
    w = get_workload(name)
    case = Case(w.seqs, w.max_tokens_per_mb)
    rng = np.random.default_rng(0)
    try:
        trees = range(len(case.ref.trees)) if n_trees is None else range(min(n_trees, len(case.ref.trees)))
        for t in trees:
            tree = case.ref.trees[t]
            print(f"fwd sampled: {name} tree={t} Np={tree.n_padded}", flush=True)
            q, k, v = attn_inputs(tree.n_padded, w.hq, w.hkv, w.head_dim, w.dtype, w.seed * 100 + t)
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, case.metas[t])
            rows = sorted(set(rng.integers(0, tree.n_padded, size=n_rows).tolist())
                          | {0, tree.n_tokens - 1, tree.n_padded - 1})
            heads = sorted(set(rng.integers(0, w.hq, size=6).tolist()) | {0, w.hq - 1})
            qh, kh, vh = host32(q), host32(k), host32(v)
            ref = oracle.attn_fwd_rows(tree, qh, kh, vh, rows, heads)
            oh, lh = host32(o), host32(lse)
            got = np.array([oh[i, h] for (i, h) in ref])
            exp = np.array([x[0] for x in ref.values()])
            assert_close(got, exp, w.dtype, f"O[{name}]")
            assert_close(np.array([lh[h, i] for (i, h) in ref]),
                         np.array([x[1] for x in ref.values()]), w.dtype, f"LSE[{name}]")
    finally:
        case.close()


def test_fwd_grpo_sampled(gpu_lib):
    _fwd_sampled(gpu_lib, "grpo")


def test_fwd_long_sampled(gpu_lib):
    _fwd_sampled(gpu_lib, "long", n_rows=24)


# ---------------------------------------------------------------- backward

def _bwd_full(gpu_lib, seqs, cap, hq, hkv, d, dtype, seed, scale=None, term_bound=False):
    case = Case(seqs, cap)
    try:
        for t, tree in enumerate(case.ref.trees):
            print(f"bwd case: dtype={dtype} hq={hq} hkv={hkv} d={d} scale={scale} tree={t} "
                  f"Np={tree.n_padded}", flush=True)
            q, k, v, do = attn_inputs(tree.n_padded, hq, hkv, d, dtype, seed + t, with_dout=True)
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, case.metas[t], softmax_scale=scale)
            dq, dk, dv = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, case.metas[t], softmax_scale=scale)
            args = (tree, host(q), host(k), host(v), host(do))
            rdq, rdk, rdv = oracle.attn_bwd(*args, scale=scale)
            mdq, mdk, mdv = (oracle.attn_bwd_magnitudes(*args, scale=scale)
                             if dtype == "f32" or term_bound else (None,) * 3)
            assert_close(host(dq), rdq, dtype, "dQ", grad=True, mag=mdq)
            assert_close(host(dk), rdk, dtype, "dK", grad=True, mag=mdk)
            assert_close(host(dv), rdv, dtype, "dV", grad=True, mag=mdv)
    finally:
        case.close()


def test_bwd_worked_example(gpu_lib):
    _bwd_full(gpu_lib, worked_example_edge(), 128, 2, 1, 64, "f32", 31)
    _bwd_full(gpu_lib, worked_example(), 128, 4, 2, 128, "bf16", 32)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 8, 2, 128),
                                             ("bf16", 5, 1, 64), ("bf16", 6, 6, 128),
                                             ("bf16", 10, 2, 128), ("bf16", 12, 2, 128),
                                             ("bf16", 6, 2, 128), ("bf16", 20, 2, 128)])
def test_bwd_several_tiles(gpu_lib, dtype, hq, hkv, d):
    """Group sizes 4 (dQ in units), 1 and 3 (blocks only), 5 and 6 (units
    for four heads of each group, blocks for the rest), 10 (two units of
    four heads per group, blocks for the last two).  At 10 heads per group
    every dK/dV entry sums ten heads' separately rounded contributions, so
    its bf16 error follows their sizes rather than |ref|: held to the term
    magnitudes (measured 0.05 % of them for dK, 0.5 % for dV)."""
    rng = np.random.default_rng(hq * 13 + d)
    seqs = prompt_groups(rng, 3, 150, 3, 20, 260)
    _bwd_full(gpu_lib, seqs, 1024, hq, hkv, d, dtype, 40 + hq, term_bound=hq // hkv > 8)


@pytest.mark.parametrize("dtype,hq,hkv,d,scale", [
    ("bf16", 10, 2, 128, 1.0), ("bf16", 10, 2, 128, 0.02),
    ("bf16", 4, 2, 64, 1.0), ("bf16", 4, 2, 64, 0.02),
    ("f32", 4, 2, 64, 0.02)])
def test_fwd_bwd_softmax_scale(gpu_lib, dtype, hq, hkv, d, scale):
    """bf16 head_dim 128 (units of four heads plus 128-query blocks of the
    fifth) at softmax scales far from 1/sqrt(d).  At 1.0 the scores span
    tens of units in the exp2 domain, so a row's running maximum grows past
    the forward's lazy-rescale threshold (2^8) about once per row after its
    first block and the rescale of O and of the row sums runs; at the
    default scale on N(0, 1) inputs it never does.  At 0.02 the softmax is
    nearly flat.  The gradients are held to their term magnitudes: at 1.0
    the softmax is peaked, dP - D cancels on the dominant keys, and the
    rounding of the bf16 O that D is formed from reaches gradients an
    absolute floor does not cover (measured: at most 0.12 %, 0.19 % and
    0.83 % of the term magnitudes for dQ, dK and dV).  The fp32 and bf16
    head_dim-64 kernels take the scale through code of their own (they
    rescale at every step).  fp32 runs at the small scale only: above the
    default its O carries the float32 rounding of the scores (u times
    scale |q||k|) times sum_j P |v|, which exceeds the 1e-5 relative bound
    of fp32 outputs on entries that cancel (measured 3.5e-6 absolute on
    |O| = 0.03 at 0.3, 3.3e-5 relative at 1.0)."""
    rng = np.random.default_rng(77)
    seqs = prompt_groups(rng, 3, 150, 3, 20, 260)
    _fwd_full(gpu_lib, seqs, 1024, hq, hkv, d, dtype, 60, scale=scale)
    _bwd_full(gpu_lib, seqs, 1024, hq, hkv, d, dtype, 61, scale=scale, term_bound=True)


def test_bwd_single_long_chain(gpu_lib):
    _bwd_full(gpu_lib, [np.arange(1, 513, dtype=np.int32)], 512, 8, 2, 128, "bf16", 45)


def test_bwd_deterministic(gpu_lib):
    import torch
    rng = np.random.default_rng(9)
    seqs = prompt_groups(rng, 2, 200, 4, 50, 300)
    case = Case(seqs, 2048)
    try:
        tree = case.ref.trees[0]
        q, k, v, do = attn_inputs(tree.n_padded, 8, 2, 128, "bf16", 50, with_dout=True)
        o, lse = gpu_lib.tree_attn_fwd(q, k, v, case.metas[0])
        a = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, case.metas[0])
        b = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, case.metas[0])
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    finally:
        case.close()


def _forest_inputs(w, sizes, with_dout=True):
    """Q, K, V (and dO) of a whole forest, trees back to back, each tree's
    rows drawn from their own seed (the layout of the forest-level metadata)."""
    import torch
    parts = [attn_inputs(s, w.hq, w.hkv, w.head_dim, w.dtype, w.seed * 100 + t, with_dout=with_dout)
             for t, s in enumerate(sizes)]
    return [torch.cat([p[n] for p in parts]).contiguous() for n in range(len(parts[0]))]


def _fwd_bwd_forest_sampled(gpu_lib, name, n_rows, n_keys, extra_keys=None):
    """One forest-level forward and backward launch over every tree of a
    full-size workload; then, tree by tree, O and LSE on sampled rows and
    heads, dQ on sampled rows, and dK/dV on sampled deep keys (whose visible
    queries the oracle enumerates one by one) for the first and last
    key/value groups.  extra_keys(tree) adds keys to check in the last tree
    (e.g. shared-prompt keys that sum over thousands of queries)."""
    w = get_workload(name)
    case = Case(w.seqs, w.max_tokens_per_mb)
    rng = np.random.default_rng(w.seed)
    fmeta = None
    try:
        sizes = [t.n_padded for t in case.ref.trees]
        fmeta = gpu_lib.forest_meta_create(case.forest)
        assert fmeta.n_padded == sum(sizes)
        print(f"fwd+bwd forest: {name} trees={len(sizes)} Np={sum(sizes)}", flush=True)
        q, k, v, do = _forest_inputs(w, sizes)
        o, lse = gpu_lib.tree_attn_fwd(q, k, v, fmeta)
        dq, dk, dv = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, fmeta)
        G = w.hq // w.hkv
        r0 = 0
        for t, tree in enumerate(case.ref.trees):
            sl = slice(r0, r0 + tree.n_padded)
            r0 += tree.n_padded
            print(f"  check: {name} tree={t} Np={tree.n_padded}", flush=True)
            qh, kh, vh, doh = (host32(x[sl]) for x in (q, k, v, do))
            oh, lh = host32(o[sl]), host32(lse[:, sl])
            dqh, dkh, dvh = host32(dq[sl]), host32(dk[sl]), host32(dv[sl])
            rows = sorted(set(rng.integers(0, tree.n_tokens, size=n_rows).tolist())
                          | {0, tree.n_tokens - 1, tree.n_padded - 1})
            heads = sorted(set(rng.integers(0, w.hq, size=4).tolist()) | {0, w.hq - 1})
            ref = oracle.attn_fwd_rows(tree, qh, kh, vh, rows, heads)
            assert_close(np.array([oh[i, h] for (i, h) in ref]), np.array([x[0] for x in ref.values()]),
                         w.dtype, f"O[{name} tree {t}]")
            assert_close(np.array([lh[h, i] for (i, h) in ref]), np.array([x[1] for x in ref.values()]),
                         w.dtype, f"LSE[{name} tree {t}]")
            se = tree.subtree_end
            deep = [j for j in range(tree.n_tokens) if se[j] - j < 40]
            keys = sorted(rng.choice(deep, size=min(n_keys, len(deep)), replace=False).tolist())
            keys.append(tree.n_padded - 1)
            if extra_keys is not None and t == len(case.ref.trees) - 1:
                keys = sorted(set(keys) | set(extra_keys(tree)))
            qrows = sorted(rng.integers(0, tree.n_tokens, size=max(n_rows // 8, 2)).tolist())
            for g in (0, w.hkv - 1):
                hs = list(range(g * G, (g + 1) * G))
                rq, rkv = oracle.attn_bwd_rows(tree, qh, kh, vh, doh, qrows, keys, (g, hs))
                assert_close(np.array([dqh[i, h] for (i, h) in rq]), np.array(list(rq.values())),
                             w.dtype, f"dQ[{name} tree {t}]", grad=True)
                assert_close(np.array([dkh[j, gg] for (j, gg) in rkv]),
                             np.array([x[0] for x in rkv.values()]), w.dtype,
                             f"dK[{name} tree {t}]", grad=True)
                assert_close(np.array([dvh[j, gg] for (j, gg) in rkv]),
                             np.array([x[1] for x in rkv.values()]), w.dtype,
                             f"dV[{name} tree {t}]", grad=True)
    finally:
        if fmeta is not None:
            import torch
            torch.cuda.synchronize()
            fmeta.destroy()
        case.close()


def test_fwd_bwd_agentic_sampled(gpu_lib):
    """Full-size agentic trees (32 query heads over 8 key/value heads: units
    only in the forward and dQ)."""
    _fwd_bwd_forest_sampled(gpu_lib, "agentic", n_rows=32, n_keys=8)


def test_fwd_bwd_bimodal_sampled(gpu_lib):
    """Full-size bimodal forest, all 23 trees in one launch (40 query heads
    over 8: the forward and dQ run units of four heads plus 128-query blocks
    for the fifth head of every group); in the last tree also the first key
    (the prompt's root, seen by every token of the tree) and a later prompt
    key, whose dK/dV sum over thousands of queries."""
    _fwd_bwd_forest_sampled(gpu_lib, "bimodal", n_rows=16, n_keys=2,
                            extra_keys=lambda tree: [0, 100])


def test_fwd_bwd_long_sampled(gpu_lib):
    """Full-size long trees (up to 32 768 tokens, 64 query heads over 8)."""
    _fwd_bwd_forest_sampled(gpu_lib, "long", n_rows=16, n_keys=3)


def test_fwd_bwd_long_control_sampled(gpu_lib):
    """The no-sharing control of the long workload: every tree is a set of
    unrelated sequences, so tree attention is varlen causal attention."""
    _fwd_bwd_forest_sampled(gpu_lib, "long_control", n_rows=12, n_keys=2)


def test_invalid_shapes_rejected(gpu_lib):
    import torch
    case = Case(worked_example(), 128)
    try:
        q, k, v = attn_inputs(128, 6, 4, 128, "bf16", 1)
        with pytest.raises(gpu_lib.PstError) as e:
            gpu_lib.tree_attn_fwd(q, k, v, case.metas[0])
        assert e.value.name == "PST_ESHAPE"
        q, k, v = attn_inputs(128, 4, 2, 96, "bf16", 1)
        with pytest.raises(gpu_lib.PstError):
            gpu_lib.tree_attn_fwd(q, k, v, case.metas[0])
        q, k, v = attn_inputs(128, 4, 2, 64, "bf16", 1)
        with pytest.raises(TypeError):
            gpu_lib.tree_attn_fwd(q.half(), k.half(), v.half(), case.metas[0])
        torch.cuda.synchronize()
    finally:
        case.close()


@pytest.mark.parametrize("hq", [8, 10])
def test_forest_meta_matches_per_tree(gpu_lib, hq):
    """One launch over the whole forest (trees back to back) gives bitwise
    the same outputs and gradients as one launch per tree (4 and 5 query
    heads per key/value head)."""
    import torch
    rng = np.random.default_rng(21)
    seqs = prompt_groups(rng, 5, 200, 3, 30, 300)
    case = Case(seqs, 512)
    try:
        assert len(case.ref.trees) >= 3
        fmeta = gpu_lib.forest_meta_create(case.forest)
        Np = sum(t.n_padded for t in case.ref.trees)
        assert fmeta.n_padded == Np
        q, k, v, do = attn_inputs(Np, hq, 2, 128, "bf16", 60, with_dout=True)
        o, lse = gpu_lib.tree_attn_fwd(q, k, v, fmeta)
        dq, dk, dv = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, fmeta)
        r0 = 0
        for t, tree in enumerate(case.ref.trees):
            sl = slice(r0, r0 + tree.n_padded)
            qs, ks, vs, dos = (x[sl].contiguous() for x in (q, k, v, do))
            ot, lt = gpu_lib.tree_attn_fwd(qs, ks, vs, case.metas[t])
            dqt, dkt, dvt = gpu_lib.tree_attn_bwd(qs, ks, vs, ot, lt, dos, case.metas[t])
            torch.cuda.synchronize()
            assert torch.equal(o[sl], ot) and torch.equal(lse[:, sl], lt)
            assert torch.equal(dq[sl], dqt) and torch.equal(dk[sl], dkt) and torch.equal(dv[sl], dvt)
            r0 += tree.n_padded
        torch.cuda.synchronize()
        fmeta.destroy()
    finally:
        case.close()

def _degenerate_inputs():
    """Single-token sequences (two of them identical, one a prefix of longer
    sequences), and trees of exactly 128 tokens (no pad rows) and of 129
    (one real row in a second block, 127 pad rows)."""
    rng = np.random.default_rng(77)
    singles = [np.array([5], np.int32), np.array([5], np.int32), np.array([9], np.int32),
               np.array([3], np.int32), np.array([3, 4, 5, 6], np.int32), np.array([3, 4], np.int32)]
    return [(singles, 128),
            ([rng.integers(0, 500, 128).astype(np.int32)], 128),
            ([rng.integers(0, 500, 129).astype(np.int32)], 256)]


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 8, 2, 128),
                                             ("bf16", 10, 2, 128)])
def test_fwd_bwd_degenerate_inputs(gpu_lib, dtype, hq, hkv, d):
    for i, (seqs, cap) in enumerate(_degenerate_inputs()):
        _fwd_full(gpu_lib, seqs, cap, hq, hkv, d, dtype, 90 + i)
        _bwd_full(gpu_lib, seqs, cap, hq, hkv, d, dtype, 95 + i)


def test_output_buffers_checked(gpu_lib):
    """Caller-supplied outputs of the wrong shape, dtype or device, and
    inputs of mixed dtypes, are refused in the binding before any launch:
    the library receives bare pointers and would write past a short buffer."""
    import torch
    case = Case(worked_example(), 128)
    try:
        m = case.metas[0]
        q, k, v, do = attn_inputs(128, 4, 2, 128, "bf16", 1, with_dout=True)
        bad = [
            dict(out=torch.empty(128, 4, 64, dtype=torch.bfloat16, device="cuda")),
            dict(out=torch.empty(128, 4, 128, dtype=torch.float32, device="cuda")),
            dict(lse=torch.empty(4, 128, dtype=torch.bfloat16, device="cuda")),
            dict(lse=torch.empty(4, 64, dtype=torch.float32, device="cuda")),
            dict(out=torch.empty(128, 4, 128, dtype=torch.bfloat16)),
        ]
        for kw in bad:
            with pytest.raises(ValueError):
                gpu_lib.tree_attn_fwd(q, k, v, m, **kw)
        o, lse = gpu_lib.tree_attn_fwd(q, k, v, m)
        for kw in (dict(dq=torch.empty_like(k)), dict(dk=torch.empty_like(q)),
                   dict(dv=torch.empty_like(v, dtype=torch.float32))):
            with pytest.raises(ValueError):
                gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, m, **kw)
        with pytest.raises(TypeError):
            gpu_lib.tree_attn_bwd(q, k, v, o.float(), lse, do, m)
        with pytest.raises(ValueError):
            gpu_lib.tree_attn_bwd(q, k, v, o, lse.to(torch.bfloat16), do, m)
        logits = torch.zeros(128, 16, dtype=torch.bfloat16, device="cuda")
        for kw in (dict(logprobs=torch.empty(m.n_out - 1, device="cuda")),
                   dict(entropy=torch.empty(m.n_out, dtype=torch.float64, device="cuda")),
                   dict(row_stats=torch.empty(128, 3, device="cuda"))):
            with pytest.raises(ValueError):
                gpu_lib.gather_tree_logprobs_entropy(logits, m, **kw)
        dl = torch.zeros(m.n_out, device="cuda")
        with pytest.raises(ValueError):
            gpu_lib.gather_tree_logprobs_entropy_bwd(logits, m, dl, dl,
                                                     dlogits=torch.empty(128, 8, dtype=torch.bfloat16,
                                                                         device="cuda"))
        torch.cuda.synchronize()
    finally:
        case.close()


def test_forest_meta_update_matches_fresh(gpu_lib):
    """One metadata object re-uploaded in place for three different forests
    (growing, then shrinking), with each forest's forward, backward and
    gather queued right after its update and no synchronization in between:
    every result equals, bit for bit, the one computed with fresh metadata
    of that forest (stream order keeps each upload behind the kernels that
    read the previous one; the two pinned staging buffers alternate)."""
    import torch
    rng = np.random.default_rng(31)
    seq_sets = [prompt_groups(rng, 2, 150, 3, 20, 200), prompt_groups(rng, 4, 300, 4, 50, 500),
                prompt_groups(rng, 1, 60, 2, 10, 40)]
    forests = [gpu_lib.build_tree(s, 1024) for s in seq_sets]
    meta = gpu_lib.forest_meta_create(forests[0])
    results, inputs = [], []
    try:
        for i, f in enumerate(forests):
            if i:
                meta.update(f)
            Np = meta.n_padded
            print(f"meta update case {i}: Np={Np}", flush=True)
            q, k, v, do = attn_inputs(Np, 8, 2, 128, "bf16", 80 + i, with_dout=True)
            logits = torch.randn(Np, 1024, device="cuda").to(torch.bfloat16)
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, meta)
            grads = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, meta)
            lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, meta)
            results.append((o, lse, *grads, lp, ent))
            inputs.append((q, k, v, do, logits))
        torch.cuda.synchronize()
        for f, (q, k, v, do, logits), got in zip(forests, inputs, results):
            fresh = gpu_lib.forest_meta_create(f)
            o, lse = gpu_lib.tree_attn_fwd(q, k, v, fresh)
            grads = gpu_lib.tree_attn_bwd(q, k, v, o, lse, do, fresh)
            lp, ent = gpu_lib.gather_tree_logprobs_entropy(logits, fresh)
            torch.cuda.synchronize()
            for a, b in zip(got, (o, lse, *grads, lp, ent)):
                assert torch.equal(a, b)
            fresh.destroy()
    finally:
        torch.cuda.synchronize()
        meta.destroy()
        for f in forests:
            f.close()
