"""Oracle: tree attention forward and backward (test infrastructure only).

The tree-training page (section "树构建过程", the attention-mask column of its
figure) fixes the rule: a packed token attends only to its ancestors, itself
included.  The Megatron integration (section "Megatron 引擎") states this as a
dense attention-mask tensor; this module builds exactly that mask by walking
parent chains and applies ordinary masked softmax attention to it, in float64.

Readings of what the page leaves open:
  * softmax scale 1/sqrt(head_dim) unless given;
  * grouped-query attention: query head h reads key/value head h // (Hq/Hkv);
  * LSE is the natural-log log-sum-exp of the scaled scores, laid out [Hq, Np];
  * a pad row sees only itself (so its output is its own value row).

Arrays: q [Np, Hq, d], k and v [Np, Hkv, d]; any real dtype, computed in float64.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .tree import Tree


def ancestors(tree: Tree, i: int) -> np.ndarray:
    """Keys visible to query i: its parent chain, itself included, ascending.
    A pad row sees only itself."""
    chain = []
    j = i
    if i >= tree.n_tokens:
        return np.array([i], dtype=np.int64)
    while j != -1:
        chain.append(j)
        j = int(tree.parent[j])
    return np.array(chain[::-1], dtype=np.int64)


def dense_mask(tree: Tree) -> np.ndarray:
    """M[i, j] = True iff key j is on query i's parent chain (i included)."""
    Np = tree.n_padded
    M = np.zeros((Np, Np), dtype=bool)
    for i in range(Np):
        M[i, ancestors(tree, i)] = True
    return M


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def _group(hq: int, hkv: int) -> int:
    if hq % hkv:
        raise ValueError(f"Hq={hq} is not a multiple of Hkv={hkv}")
    return hq // hkv


def _logsumexp(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True)))[..., 0]


def attn_fwd(tree: Tree, q, k, v, scale=None, mask=None):
    """O[i,h] = sum_j softmax_j(scale * q[i,h] . k[j,g]) v[j,g] over visible j.
    Returns (O [Np,Hq,d] float64, LSE [Hq,Np] float64)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    Np, hq, d = q.shape
    G = _group(hq, k.shape[1])
    s = _scale(d, scale)
    M = dense_mask(tree) if mask is None else mask
    O = np.zeros_like(q)
    LSE = np.zeros((hq, Np))
    for h in range(hq):
        g = h // G
        S = s * (q[:, h, :] @ k[:, g, :].T)
        S = np.where(M, S, -np.inf)
        lse = _logsumexp(S)
        P = np.exp(S - lse[:, None])
        O[:, h, :] = P @ v[:, g, :]
        LSE[h] = lse
    return O, LSE


def attn_bwd(tree: Tree, q, k, v, dout, scale=None, mask=None):
    """Gradients of sum(dout * O) with respect to q, k, v (float64): the
    softmax-attention vector-Jacobian product restricted to the tree mask;
    each key/value head sums the contributions of the query heads that read it."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    Np, hq, d = q.shape
    G = _group(hq, k.shape[1])
    s = _scale(d, scale)
    M = dense_mask(tree) if mask is None else mask
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(hq):
        g = h // G
        S = np.where(M, s * (q[:, h, :] @ k[:, g, :].T), -np.inf)
        P = np.exp(S - _logsumexp(S)[:, None])
        O = P @ v[:, g, :]
        Drow = (dout[:, h, :] * O).sum(axis=1)
        dv[:, g, :] += P.T @ dout[:, h, :]
        dP = dout[:, h, :] @ v[:, g, :].T
        dS = P * (dP - Drow[:, None])
        dq[:, h, :] = s * (dS @ k[:, g, :])
        dk[:, g, :] += s * (dS.T @ q[:, h, :])
    return dq, dk, dv


def attn_bwd_magnitudes(tree: Tree, q, k, v, dout, scale=None, mask=None):
    """The backward of attn_bwd with every elementary product taken by
    absolute value, down to the dot products inside dP and D:

        A_ij    = sum_c |dO_ic| |V_jc|              (bounds |dP_ij|, dP = dO.V^T)
        B_i     = sum_c |dO_ic| sum_j P_ij |V_jc|   (bounds |D_i|, D = rowsum(dO*O))
        mdQ[i]  = s * sum_j P_ij (A_ij + B_i) |K_j|
        mdK[j]  = s * sum_i P_ij (A_ij + B_i) |Q_i|
        mdV[j]  = sum_i P_ij |dO_i|

    (P >= 0 needs no bars).  Each entry is the sum of the sizes of all the
    products that the gradient entry is built from, so |dQ| <= mdQ and so
    on, and the rounding of a computed value is at most a small multiple of
    the unit roundoff times this magnitude.  dS = P (dP - D) cancels (a token
    that sees only itself has dP = D exactly), and so can the dot products
    inside dP and D; where they do, the gradient is far smaller than its
    terms, and only the magnitude says how large a computed value's rounding
    may be.  float64, same shapes as attn_bwd."""
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    Np, hq, d = q.shape
    G = _group(hq, k.shape[1])
    s = _scale(d, scale)
    M = dense_mask(tree) if mask is None else mask
    mq, mk, mv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(hq):
        g = h // G
        S = np.where(M, s * (q[:, h, :] @ k[:, g, :].T), -np.inf)
        P = np.exp(S - _logsumexp(S)[:, None])
        adO, aV = np.abs(dout[:, h, :]), np.abs(v[:, g, :])
        A = adO @ aV.T
        B = (adO * (P @ aV)).sum(axis=1)
        W = P * (A + B[:, None])
        mv[:, g, :] += P.T @ adO
        mq[:, h, :] = s * (W @ np.abs(k[:, g, :]))
        mk[:, g, :] += s * (W.T @ np.abs(q[:, h, :]))
    return mq, mk, mv


def attn_fwd_rows(tree: Tree, q, k, v, rows: Iterable[int], heads: Iterable[int],
                  scale=None):
    """The forward definition evaluated for selected (row, head) pairs only,
    walking each row's parent chain.  Returns {(i, h): (o [d], lse)}."""
    d = q.shape[2]
    G = _group(q.shape[1], k.shape[1])
    s = _scale(d, scale)
    out = {}
    for i in rows:
        anc = ancestors(tree, int(i))
        for h in heads:
            g = h // G
            qi = np.asarray(q[i, h, :], dtype=np.float64)
            kk = np.asarray(k[anc, g, :], dtype=np.float64)
            vv = np.asarray(v[anc, g, :], dtype=np.float64)
            sc = s * (kk @ qi)
            m = sc.max()
            e = np.exp(sc - m)
            out[(int(i), int(h))] = (e @ vv / e.sum(), m + math.log(e.sum()))
    return out


def attn_bwd_rows(tree: Tree, q, k, v, dout, dq_rows: Iterable[int],
                  dkv_rows: Iterable[int], heads_of_group, scale=None):
    """Backward definition for selected rows.

    dq_rows: queries i for which dQ[i, h] is wanted, h in `heads_of_group`'s heads.
    dkv_rows: keys j for which dK[j, g], dV[j, g] are wanted (g the group).
    heads_of_group: (g, [query heads of group g]).
    Every query that sees a requested key is evaluated from its parent chain.
    Returns ({(i,h): dq}, {(j,g): (dk, dv)})."""
    d = q.shape[2]
    s = _scale(d, scale)
    g, heads = heads_of_group
    f64 = lambda x: np.asarray(x, dtype=np.float64)  # noqa: E731

    anc_of, terms = {}, {}

    def row_terms(i, h):
        # each (query, head) is evaluated once, however many requested keys it sees
        if (i, h) not in terms:
            if i not in anc_of:
                anc_of[i] = ancestors(tree, i)
            anc = anc_of[i]
            qi, doi = f64(q[i, h, :]), f64(dout[i, h, :])
            kk, vv = f64(k[anc, g, :]), f64(v[anc, g, :])
            sc = s * (kk @ qi)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            o = p @ vv
            dp = vv @ doi
            ds = p * (dp - doi @ o)
            terms[(i, h)] = (anc, p, ds, qi, doi)
        return terms[(i, h)]

    dq = {}
    for i in dq_rows:
        for h in heads:
            anc, p, ds, qi, doi = row_terms(int(i), h)
            dq[(int(i), h)] = s * (ds @ f64(k[anc, g, :]))
    kids = {}
    for i in range(tree.n_tokens):
        kids.setdefault(int(tree.parent[i]), []).append(i)
    dkv = {}
    for j in dkv_rows:
        j = int(j)
        dk_j, dv_j = np.zeros(d), np.zeros(d)
        # queries that see key j: j itself and every real token below it
        seers, frontier = [j], [j]
        while frontier and j < tree.n_tokens:
            frontier = [c for x in frontier for c in kids.get(x, ())]
            seers.extend(frontier)
        for i in seers:
            for h in heads:
                anc, p, ds, qi, doi = row_terms(i, h)
                pos = int(np.nonzero(anc == j)[0][0])
                dv_j += p[pos] * doi
                dk_j += s * ds[pos] * qi
        dkv[(j, g)] = (dk_j, dv_j)
    return dq, dkv
