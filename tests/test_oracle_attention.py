"""Pins of the oracle's tree attention (CPU only).

 * the invariant that defines tree attention: every packed token's output
   equals plain causal attention over its own unpacked sequence (torch CPU
   scaled_dot_product_attention, float64);
 * closed forms: constant values give O = V; depth-0 and pad tokens see only
   themselves;
 * backward: central finite differences in float64, and torch CPU autograd of
   per-sequence causal attention mapped back through the index maps;
 * the row-sampling forms agree with the dense forms.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import worked_example, worked_example_edge


def _tree_inputs(tree, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    Np = tree.n_padded
    q = rng.standard_normal((Np, hq, d))
    k = rng.standard_normal((Np, hkv, d))
    v = rng.standard_normal((Np, hkv, d))
    do = rng.standard_normal((Np, hq, d))
    return q, k, v, do


def _random_seqs(rng, n_groups=3):
    seqs = []
    for _ in range(n_groups):
        prompt = rng.integers(0, 3, size=int(rng.integers(1, 40)))
        for _ in range(int(rng.integers(1, 4))):
            resp = rng.integers(0, 3, size=int(rng.integers(1, 60)))
            seqs.append(np.concatenate([prompt, resp]).astype(np.int32))
    return seqs


def _causal_per_seq(tree, seq_ids, q, k, v, scale=None):
    """torch CPU causal attention on each unpacked sequence, inputs gathered
    from the packed rows."""
    hq, hkv = q.shape[1], k.shape[1]
    out = {}
    for sid in seq_ids:
        idx = torch.as_tensor(tree.seq_index[sid], dtype=torch.long)
        Q = torch.as_tensor(q)[idx].permute(1, 0, 2)          # [hq, L, d]
        K = torch.as_tensor(k)[idx].permute(1, 0, 2)
        V = torch.as_tensor(v)[idx].permute(1, 0, 2)
        K = K.repeat_interleave(hq // hkv, dim=0)
        V = V.repeat_interleave(hq // hkv, dim=0)
        O = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        out[sid] = O.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("hq,hkv,d", [(2, 2, 16), (4, 1, 8), (6, 2, 32)])
def test_fwd_equals_causal_per_sequence(hq, hkv, d):
    rng = np.random.default_rng(hq * 100 + d)
    for trial in range(3):
        seqs = _random_seqs(rng)
        f = oracle.build_forest(seqs, 256)
        for tree in f.trees:
            q, k, v, _ = _tree_inputs(tree, hq, hkv, d, trial)
            O, LSE = oracle.attn_fwd(tree, q, k, v)
            ref = _causal_per_seq(tree, tree.seq_ids, q, k, v)
            for sid in tree.seq_ids:
                np.testing.assert_allclose(O[tree.seq_index[sid]], ref[sid], rtol=1e-12, atol=1e-12)


def test_fwd_worked_example_and_scale():
    for seqs in (worked_example(), worked_example_edge()):
        tree = oracle.build_forest(seqs, 128).trees[0]
        q, k, v, _ = _tree_inputs(tree, 2, 1, 8, 3)
        O, _ = oracle.attn_fwd(tree, q, k, v, scale=0.3)
        ref = _causal_per_seq(tree, tree.seq_ids, q, k, v, scale=0.3)
        for sid in tree.seq_ids:
            np.testing.assert_allclose(O[tree.seq_index[sid]], ref[sid], rtol=1e-12, atol=1e-12)


def test_fwd_closed_forms():
    tree = oracle.build_forest(_random_seqs(np.random.default_rng(5)), 256).trees[0]
    q, k, v, _ = _tree_inputs(tree, 4, 2, 16, 0)
    # constant values: every convex combination returns the constant
    vc = np.broadcast_to(np.arange(16.0), v.shape).copy()
    O, _ = oracle.attn_fwd(tree, q, k, vc)
    np.testing.assert_allclose(O, np.broadcast_to(np.arange(16.0), O.shape), atol=1e-12)
    # depth-0 tokens and pads see only themselves
    O, LSE = oracle.attn_fwd(tree, q, k, v)
    solo = [i for i in range(tree.n_padded) if i >= tree.n_tokens or tree.parent[i] == -1]
    for i in solo:
        for h in range(4):
            g = h // 2
            np.testing.assert_allclose(O[i, h], v[i, g], atol=1e-12)
            assert LSE[h, i] == pytest.approx(q[i, h] @ k[i, g] / 4.0, abs=1e-12)


def test_fwd_rows_match_dense():
    tree = oracle.build_forest(_random_seqs(np.random.default_rng(6)), 256).trees[0]
    q, k, v, _ = _tree_inputs(tree, 4, 2, 16, 1)
    O, LSE = oracle.attn_fwd(tree, q, k, v)
    rows = [0, 5, tree.n_tokens - 1, tree.n_padded - 1]
    got = oracle.attn_fwd_rows(tree, q, k, v, rows, range(4))
    for (i, h), (o, lse) in got.items():
        np.testing.assert_allclose(o, O[i, h], atol=1e-12)
        assert lse == pytest.approx(LSE[h, i], abs=1e-12)


def test_bwd_finite_differences():
    seqs = worked_example_edge() + [np.array([1, 2, 3, 9, 9], np.int32)]
    tree = oracle.build_forest(seqs, 128).trees[0]
    hq, hkv, d = 4, 2, 3
    q, k, v, do = _tree_inputs(tree, hq, hkv, d, 7)
    dq, dk, dv = oracle.attn_bwd(tree, q, k, v, do)

    def loss(q, k, v):
        O, _ = oracle.attn_fwd(tree, q, k, v)
        return float((O * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    N = tree.n_tokens
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        picks = [(int(rng.integers(0, N)), int(rng.integers(0, arr.shape[1])), int(rng.integers(0, d)))
                 for _ in range(12)] + [(N + 2, 0, 1)]     # one pad row
        for (i, h, c) in picks:
            a1, a2 = arr.copy(), arr.copy()
            a1[i, h, c] += eps
            a2[i, h, c] -= eps
            args1 = {"q": q, "k": k, "v": v}
            args2 = dict(args1)
            args1[name], args2[name] = a1, a2
            fd = (loss(**args1) - loss(**args2)) / (2 * eps)
            assert grad[i, h, c] == pytest.approx(fd, abs=1e-7, rel=1e-6), (name, i, h, c)


@pytest.mark.parametrize("hq,hkv,scale", [(2, 2, None), (4, 1, None), (6, 3, None),
                                          (4, 2, 1.0), (4, 2, 0.05)])
def test_bwd_equals_autograd_of_causal(hq, hkv, scale):
    """Loss = sum over packed real rows of <dO_i, O_i>.  Each packed row is
    represented by one (sequence, position) that reaches it; autograd through
    the per-sequence causal attention and the index gathers must give the
    packed gradients, at the default softmax scale and at others.  Pad rows:
    dV = dO, dQ = dK = 0."""
    rng = np.random.default_rng(hq + 10 * hkv)
    d = 8
    seqs = _random_seqs(rng)
    tree = oracle.build_forest(seqs, 256).trees[0]
    q, k, v, do = _tree_inputs(tree, hq, hkv, d, 2)
    dq, dk, dv = oracle.attn_bwd(tree, q, k, v, do, scale=scale)
    N = tree.n_tokens
    Q = torch.tensor(q, requires_grad=True)
    K = torch.tensor(k, requires_grad=True)
    V = torch.tensor(v, requires_grad=True)
    owner = {}
    for sid in tree.seq_ids:
        for t, i in enumerate(tree.seq_index[sid]):
            owner.setdefault(int(i), (sid, t))
    loss = 0.0
    for sid in tree.seq_ids:
        idx = torch.as_tensor(tree.seq_index[sid], dtype=torch.long)
        Qs = Q[idx].permute(1, 0, 2)
        Ks = K[idx].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        Vs = V[idx].permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
        Os = F.scaled_dot_product_attention(Qs, Ks, Vs, is_causal=True, scale=scale).permute(1, 0, 2)
        w = np.zeros((len(idx), hq, d))
        for t, i in enumerate(tree.seq_index[sid]):
            if owner[int(i)] == (sid, t):
                w[t] = do[i]
        loss = loss + (Os * torch.as_tensor(w)).sum()
    loss.backward()
    np.testing.assert_allclose(dq[:N], Q.grad.numpy()[:N], atol=1e-10)
    np.testing.assert_allclose(dk[:N], K.grad.numpy()[:N], atol=1e-10)
    np.testing.assert_allclose(dv[:N], V.grad.numpy()[:N], atol=1e-10)
    G = hq // hkv
    np.testing.assert_allclose(dq[N:], 0, atol=1e-12)
    np.testing.assert_allclose(dk[N:], 0, atol=1e-12)
    np.testing.assert_allclose(dv[N:], do[N:].reshape(-1, hkv, G, d).sum(2), atol=1e-12)


def test_bwd_rows_match_dense():
    tree = oracle.build_forest(_random_seqs(np.random.default_rng(8)), 256).trees[0]
    q, k, v, do = _tree_inputs(tree, 4, 2, 8, 4)
    dq, dk, dv = oracle.attn_bwd(tree, q, k, v, do)
    for g in range(2):
        heads = [2 * g, 2 * g + 1]
        rows = [0, 3, tree.n_tokens - 1, tree.n_padded - 1]
        gq, gkv = oracle.attn_bwd_rows(tree, q, k, v, do, rows, rows, (g, heads))
        for (i, h), x in gq.items():
            np.testing.assert_allclose(x, dq[i, h], atol=1e-12)
        for (j, gg), (a, b) in gkv.items():
            np.testing.assert_allclose(a, dk[j, gg], atol=1e-12)
            np.testing.assert_allclose(b, dv[j, gg], atol=1e-12)


# ------------------------------------------------ gradient term magnitudes

def _magnitudes_brute_force(tree, q, k, v, do, s):
    """The absolute sums of the elementary products behind every gradient
    entry, by loops over each query's parent chain (no dense mask, no matrix
    products): dQ_ic sums s P_ij dO_ie V_je K_jc over visible j and every e
    (the dP terms), and s P_ij dO_ie P_ij' V_j'e K_jc over visible j, j' and
    every e (the D terms); dK and dV sum the matching products over the
    queries that see a key."""
    Np, hq, d = q.shape
    G = hq // k.shape[1]
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(Np):
        anc = oracle.ancestors(tree, i)
        for h in range(hq):
            g = h // G
            sc = np.array([s * float(np.dot(q[i, h], k[j, g])) for j in anc])
            p = np.exp(sc - sc.max())
            p /= p.sum()
            dp_abs = [sum(abs(do[i, h, e] * v[j, g, e]) for e in range(d)) for j in anc]
            d_abs = sum(abs(do[i, h, e] * p[n2] * v[j2, g, e])
                        for e in range(d) for n2, j2 in enumerate(anc))
            for n, j in enumerate(anc):
                for c in range(d):
                    mq[i, h, c] += s * p[n] * (dp_abs[n] + d_abs) * abs(k[j, g, c])
                    mk[j, g, c] += s * p[n] * (dp_abs[n] + d_abs) * abs(q[i, h, c])
                    mv[j, g, c] += p[n] * abs(do[i, h, c])
    return mq, mk, mv


@pytest.mark.parametrize("scale", [None, 1.0])
def test_bwd_magnitudes_brute_force(scale):
    tree = oracle.build_forest(worked_example_edge() + [np.array([1, 2, 9], np.int32)], 128).trees[0]
    q, k, v, do = _tree_inputs(tree, 4, 2, 3, 12)
    got = oracle.attn_bwd_magnitudes(tree, q, k, v, do, scale=scale)
    exp = _magnitudes_brute_force(tree, q, k, v, do, 1 / np.sqrt(3) if scale is None else scale)
    for a, b in zip(got, exp):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_bwd_magnitudes_bound_the_gradients():
    """|dQ| <= mdQ, |dK| <= mdK, |dV| <= mdV entrywise (triangle inequality);
    flipping the sign of dO flips the gradients and leaves the magnitudes;
    with dO >= 0 every dV term is non-negative, so mdV equals dV."""
    tree = oracle.build_forest(_random_seqs(np.random.default_rng(13)), 256).trees[0]
    q, k, v, do = _tree_inputs(tree, 4, 2, 8, 14)
    grads = oracle.attn_bwd(tree, q, k, v, do)
    mags = oracle.attn_bwd_magnitudes(tree, q, k, v, do)
    for gr, mg in zip(grads, mags):
        assert np.all(np.abs(gr) <= mg * (1 + 1e-12) + 1e-15)
    flipped = oracle.attn_bwd_magnitudes(tree, q, k, v, -do)
    for a, b in zip(mags, flipped):
        np.testing.assert_allclose(a, b, rtol=1e-13)
    pos = np.abs(do)
    dv = oracle.attn_bwd(tree, q, k, v, pos)[2]
    np.testing.assert_allclose(oracle.attn_bwd_magnitudes(tree, q, k, v, pos)[2], dv, rtol=1e-12)


def test_bwd_magnitudes_single_token():
    """A token that sees only itself (P = 1, O = V, so dP = D): dQ = dK = 0
    exactly, while the magnitudes are 2 s (|dO|.|V|) |K| and 2 s (|dO|.|V|) |Q|
    (summed over the query heads of the group for K) and |dO| for V."""
    tree = oracle.build_forest([np.array([7], np.int32)], 128).trees[0]
    q, k, v, do = _tree_inputs(tree, 2, 1, 4, 15)
    s = 0.5
    dq, dk, _ = oracle.attn_bwd(tree, q, k, v, do)
    mq, mk, mv = oracle.attn_bwd_magnitudes(tree, q, k, v, do)
    for i in (0, 5, tree.n_padded - 1):         # the real token and two pad rows
        a = [float(np.dot(np.abs(do[i, h]), np.abs(v[i, 0]))) for h in range(2)]
        np.testing.assert_allclose(dq[i], 0, atol=1e-12)
        np.testing.assert_allclose(dk[i], 0, atol=1e-12)
        for h in range(2):
            np.testing.assert_allclose(mq[i, h], 2 * s * a[h] * np.abs(k[i, 0]), rtol=1e-12)
        np.testing.assert_allclose(mk[i, 0], 2 * s * (a[0] * np.abs(q[i, 0]) + a[1] * np.abs(q[i, 1])),
                                   rtol=1e-12)
        np.testing.assert_allclose(mv[i, 0], np.abs(do[i, 0]) + np.abs(do[i, 1]), rtol=1e-12)
