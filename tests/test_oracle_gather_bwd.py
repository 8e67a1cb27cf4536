"""Pins of the oracle's gather backward (CPU only).

 * torch autograd of the roll-label computation on each unpacked sequence
   (log_softmax + gather, entropy from softmax), rows read through the index
   maps, gives the same gradient with respect to the packed logits;
 * central finite differences of the oracle's own forward agree;
 * the row-subset form equals the full form on the rows it is asked for;
 * closed forms: with uniform logits the entropy gradient vanishes
   (log p + H = 0) and a single logprob gradient g gives g (e_target - 1/V);
   pad rows and the last position of each sequence contribute nothing.
"""

import math

import numpy as np
import torch

import oracle
from workloads import worked_example, worked_example_edge


def _seqs(rng, vocab):
    seqs = []
    for _ in range(2):
        prompt = rng.integers(0, vocab, size=int(rng.integers(1, 12)))
        for _ in range(int(rng.integers(1, 4))):
            resp = rng.integers(0, vocab, size=int(rng.integers(1, 15)))
            seqs.append(np.concatenate([prompt, resp]).astype(np.int32))
    return seqs


def _autograd(tree, seqs, logits, dlp, dh):
    x = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    loss = torch.zeros((), dtype=torch.float64)
    off = 0
    for sid in tree.seq_ids:
        seq = torch.as_tensor(np.asarray(seqs[sid], dtype=np.int64))
        rows = x[torch.as_tensor(tree.seq_index[sid], dtype=torch.long)]
        logp = torch.log_softmax(rows, dim=-1)
        L = len(seq)
        lp = logp[torch.arange(L - 1), seq[1:]]
        ent = -(logp.exp() * logp).sum(-1)
        loss = loss + (torch.as_tensor(dlp[off:off + L - 1]) * lp).sum()
        loss = loss + (torch.as_tensor(dh[off:off + L]) * ent).sum()
        off += L
    loss.backward()
    return x.grad.numpy()


def test_bwd_equals_autograd():
    rng = np.random.default_rng(3)
    for vocab in (5, 17):
        seqs = _seqs(rng, vocab)
        f = oracle.build_forest(seqs, 128)
        for tree in f.trees:
            logits = rng.normal(0, 2.0, size=(tree.n_padded, vocab))
            n = int(tree.out_offsets[-1])
            dlp, dh = rng.normal(size=n), rng.normal(size=n)
            got = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, dlp, dh)
            want = _autograd(tree, seqs, logits, dlp, dh)
            assert np.abs(got - want).max() < 1e-12


def test_bwd_finite_differences():
    rng = np.random.default_rng(4)
    seqs = worked_example()
    tree = oracle.build_forest(seqs, 128).trees[0]
    V = 9
    logits = rng.normal(0, 1.0, size=(tree.n_padded, V))
    n = int(tree.out_offsets[-1])
    dlp, dh = rng.normal(size=n), rng.normal(size=n)
    g = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, dlp, dh)

    def loss(xx):
        lp, h = oracle.gather_logprobs_entropy(tree, seqs, xx)
        return float((dlp * lp).sum() + (dh * h).sum())

    eps = 1e-6
    for row in range(tree.n_tokens):
        for v in range(V):
            xp, xm = logits.copy(), logits.copy()
            xp[row, v] += eps
            xm[row, v] -= eps
            assert abs((loss(xp) - loss(xm)) / (2 * eps) - g[row, v]) < 1e-7
    assert (g[tree.n_tokens:] == 0).all()


def test_bwd_closed_forms():
    seqs = worked_example_edge()
    tree = oracle.build_forest(seqs, 128).trees[0]
    V = 20
    logits = np.full((tree.n_padded, V), 0.3)
    n = int(tree.out_offsets[-1])
    # entropy only: uniform rows are a stationary point of the entropy
    g = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, np.zeros(n), np.ones(n))
    assert np.abs(g).max() < 1e-12
    # one logprob gradient at the first position of the first sequence
    sid = tree.seq_ids[0]
    seq = np.asarray(seqs[sid])
    dlp = np.zeros(n)
    dlp[0] = 2.5
    g = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, dlp, np.zeros(n))
    row = int(tree.seq_index[sid][0])
    want = np.full(V, -2.5 / V)
    want[int(seq[1])] += 2.5
    assert np.abs(g[row] - want).max() < 1e-12
    g[row] = 0
    assert not g.any()
    # the last position's logprob is a constant: no gradient
    dlp = np.zeros(n)
    dlp[len(seq) - 1] = 1.0
    g = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, dlp, np.zeros(n))
    assert not g.any()
    assert math.isclose(float(np.log(V)), float(oracle.row_lse_entropy(logits[:1])[1][0]), rel_tol=1e-12)


def test_bwd_rows_subset_matches_full():
    rng = np.random.default_rng(5)
    seqs = _seqs(rng, 11)
    tree = oracle.build_forest(seqs, 128).trees[0]
    logits = rng.normal(0, 1.5, size=(tree.n_padded, 11))
    n = int(tree.out_offsets[-1])
    dlp, dh = rng.normal(size=n), rng.normal(size=n)
    full = oracle.gather_logprobs_entropy_bwd(tree, seqs, logits, dlp, dh)
    rows = [0, 3, tree.n_tokens - 1, tree.n_padded - 1]
    sub = oracle.gather_logprobs_entropy_bwd(tree, seqs, {r: logits[r] for r in rows}, dlp, dh,
                                             rows=rows)
    for r in rows:
        assert np.array_equal(sub[r], full[r])
