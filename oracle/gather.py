"""Oracle: per-sequence log-probabilities and entropies from packed-tree logits
(test infrastructure only).

The tree-training page (section "对数概率计算") explains why the labels cannot be
obtained by rolling input_ids: positions are shared between sequences, so each
sequence must recover its own token order from the tree.  The plain definition
is used here: for every sequence s of length L and every position t, read the
logits row of the tree token holding s[t] and take

    logprob[t] = log_softmax(row)[s[t+1]]   for t < L-1,   logprob[L-1] = 0
    entropy[t] = -sum_v p_v log p_v,        p = softmax(row)

in float64, natural logs, temperature 1.  Outputs of the sequences of one tree
are concatenated in ascending input index (the page's last step concatenates
per-sequence results).

The backward (the loss path the same section implies: training differentiates
these log-probabilities and entropies) is the plain chain rule, output by
output: with log p = x - lse and H = lse - sum p x,

    d logprob[t] / d x_v = [v = s[t+1]] - p_v          (t < L-1; 0 at t = L-1)
    d entropy[t] / d x_v = -p_v (log p_v + H)

summed over every (sequence, position) whose token's row is x; rows that no
output reads (pad rows) get zero.
"""

from __future__ import annotations

import numpy as np

from .tree import Tree


def row_lse_entropy(rows: np.ndarray):
    """log-sum-exp and entropy of each row of `rows` [n, V], in float64."""
    x = np.asarray(rows, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    p = e / z
    # a zero-probability entry adds nothing to -sum p log p (0 log 0 = 0),
    # also where its logit is -inf
    ent = lse - (p * np.where(p > 0, x, 0.0)).sum(axis=1)
    return lse, ent


def gather_logprobs_entropy(tree: Tree, seqs, logits):
    """logits: [Np, V] (any real dtype; only real rows are read).
    Returns (logprobs, entropy), float64 arrays of length sum of the tree's
    sequence lengths."""
    outs_lp, outs_h = [], []
    for sid in tree.seq_ids:
        seq = np.asarray(seqs[sid])
        idx = tree.seq_index[sid]
        x = np.asarray(logits[idx], dtype=np.float64)
        lse, ent = row_lse_entropy(x)
        lp = np.zeros(len(seq))
        nxt = seq[1:]
        lp[:-1] = x[np.arange(len(seq) - 1), nxt] - lse[:-1]
        outs_lp.append(lp)
        outs_h.append(ent)
    return np.concatenate(outs_lp), np.concatenate(outs_h)


def gather_logprobs_entropy_bwd(tree: Tree, seqs, logits, dlogprobs, dentropy, rows=None):
    """Gradient of sum(dlogprobs * logprobs + dentropy * entropy) with respect
    to the logits [Np, V] of one tree, where logprobs/entropy are
    gather_logprobs_entropy(tree, seqs, logits).  Returns float64 [Np, V].

    With `rows` (a collection of row indices), `logits` maps each of those
    rows to its logits and only their gradients are formed: a dict row ->
    float64 [V] (for trees whose full logits do not fit the host)."""
    if rows is None:
        x_all = np.asarray(logits, dtype=np.float64)
        grad = np.zeros_like(x_all)
        want = None
    else:
        want = set(int(r) for r in rows)
        grad = {r: np.zeros(len(logits[r])) for r in want}
    dlp = np.asarray(dlogprobs, dtype=np.float64)
    dh = np.asarray(dentropy, dtype=np.float64)
    off = 0
    for sid in tree.seq_ids:
        seq = np.asarray(seqs[sid])
        idx = tree.seq_index[sid]
        for t in range(len(seq)):
            row = int(idx[t])
            if want is not None and row not in want:
                continue
            x = np.asarray(logits[row], dtype=np.float64) if want is not None else x_all[row]
            m = x.max()
            e = np.exp(x - m)
            z = e.sum()
            p = e / z
            logp = x - (m + np.log(z))
            ent = -(p * np.where(p > 0, logp, 0.0)).sum()
            # entropy term; a zero-probability entry has zero derivative
            grad[row] += dh[off + t] * (-p * np.where(p > 0, logp + ent, 0.0))
            if t < len(seq) - 1:
                g = -p.copy()
                g[int(seq[t + 1])] += 1.0
                grad[row] += dlp[off + t] * g
        off += len(seq)
    return grad
