"""Pins of the oracle's logprob/entropy gather (CPU only).

 * it equals the standard roll-label computation (torch CPU log_softmax +
   gather, and entropy) on each unpacked sequence, whose logits rows are read
   through the index maps;
 * closed forms: uniform logits give logprob -log V and entropy log V; a
   dominant spike on the next token gives logprob -> 0 and entropy -> 0;
   k equal logits with the rest of the vocabulary at -inf (a masked
   vocabulary) give logprob -log k and entropy log k;
 * the worked example yields 11 outputs in sequence order, last of each 0.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import worked_example, worked_example_edge


def _seqs(rng, vocab):
    seqs = []
    for _ in range(3):
        prompt = rng.integers(0, vocab, size=int(rng.integers(1, 30)))
        for _ in range(int(rng.integers(1, 4))):
            resp = rng.integers(0, vocab, size=int(rng.integers(1, 40)))
            seqs.append(np.concatenate([prompt, resp]).astype(np.int32))
    return seqs


def test_gather_equals_roll_labels():
    rng = np.random.default_rng(0)
    for vocab in (3, 17, 300):
        seqs = _seqs(rng, vocab)
        f = oracle.build_forest(seqs, 256)
        for tree in f.trees:
            logits = rng.standard_normal((tree.n_padded, vocab)) * 2
            lp, ent = oracle.gather_logprobs_entropy(tree, seqs, logits)
            exp_lp, exp_h = [], []
            for sid in tree.seq_ids:
                x = torch.as_tensor(logits[tree.seq_index[sid]])
                logp = torch.log_softmax(x, dim=-1)
                labels = torch.as_tensor(np.roll(seqs[sid], -1).astype(np.int64))
                g = logp.gather(1, labels[:, None])[:, 0]
                g[-1] = 0.0
                exp_lp.append(g.numpy())
                exp_h.append(-(logp.exp() * logp).sum(-1).numpy())
            np.testing.assert_allclose(lp, np.concatenate(exp_lp), atol=1e-12)
            np.testing.assert_allclose(ent, np.concatenate(exp_h), atol=1e-12)


def test_gather_closed_forms():
    seqs = worked_example_edge()
    tree = oracle.build_forest(seqs, 128).trees[0]
    V = 64
    lp, ent = oracle.gather_logprobs_entropy(tree, seqs, np.full((128, V), 0.37))
    last = set((tree.out_offsets[1:] - 1).tolist())
    for p in range(len(lp)):
        assert lp[p] == (0.0 if p in last else lp[p])
        if p not in last:
            assert abs(lp[p] + math.log(V)) < 1e-12
        assert abs(ent[p] - math.log(V)) < 1e-12
    # spike on the next token: every logprob ~ 0, entropy ~ 0
    big = np.zeros((128, V))
    for sid in tree.seq_ids:
        s = seqs[sid]
        for t in range(len(s) - 1):
            big[tree.seq_index[sid][t], s[t + 1]] = 200.0
    # branch rows (A and G) have several next tokens: give them their own checks
    lp, ent = oracle.gather_logprobs_entropy(tree, seqs, big)
    for i, sid in enumerate(tree.seq_ids):
        s = seqs[sid]
        for t in range(len(s) - 1):
            p = tree.out_offsets[i] + t
            row = tree.seq_index[sid][t]
            n_next = tree.child_ptr[row + 1] - tree.child_ptr[row]
            assert abs(lp[p] + math.log(n_next)) < 1e-12


def test_gather_worked_example_layout():
    seqs = worked_example()
    tree = oracle.build_forest(seqs, 128).trees[0]
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((128, 9))
    lp, ent = oracle.gather_logprobs_entropy(tree, seqs, logits)
    assert len(lp) == len(ent) == 11
    lse, H = oracle.row_lse_entropy(logits[:8])
    # [lp(0->B), lp(1->C), lp(2->D), 0 | lp(0->B), lp(1->E), lp(4->F), 0 | lp(0->G), lp(6->H), 0]
    A, B, C, D, E, F_, G, Hh = range(1, 9)
    exp = [(0, B), (1, C), (2, D), None, (0, B), (1, E), (4, F_), None, (0, G), (6, Hh), None]
    for p, e in enumerate(exp):
        assert lp[p] == (0.0 if e is None else logits[e[0], e[1]] - lse[e[0]])
    rows = [0, 1, 2, 3, 0, 1, 4, 5, 0, 6, 7]
    np.testing.assert_allclose(ent, H[rows], atol=0)


def test_gather_masked_vocabulary_closed_form():
    """Entries at -inf have probability 0 and add nothing to the entropy."""
    V, k = 12, 5
    row = np.full((1, V), -np.inf)
    row[0, 3:3 + k] = 0.7
    lse, ent = oracle.row_lse_entropy(row)
    assert lse[0] == pytest.approx(0.7 + math.log(k), abs=1e-12)
    assert ent[0] == pytest.approx(math.log(k), abs=1e-12)
    seqs = [np.array([1, 4, 6], dtype=np.int32)]
    f = oracle.build_forest(seqs, 128)
    logits = np.full((128, V), -np.inf)
    logits[:, 3:3 + k] = 0.7
    lp, h = oracle.gather_logprobs_entropy(f.trees[0], seqs, logits)
    assert np.allclose(lp, [-math.log(k), -math.log(k), 0.0], atol=1e-12)
    assert np.allclose(h, math.log(k), atol=1e-12)
