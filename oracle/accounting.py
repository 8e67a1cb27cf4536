"""Oracle: token and FLOP accounting (test infrastructure only).

tree_token_ratio is tree tokens over original tokens (AReaL tree-training page,
section "指标和监控"); lower means more sharing.  It is taken over the real
(unpadded) tokens of all trees.  Attention work counts only visible pairs:
4 * head_dim * Hq flops per visible (query, key) pair for the forward pass (a
multiply-add in Q.K^T and in P.V); the backward pass is counted as 2.5 times
the forward pass (its five matrix products, including the recomputed Q.K^T).
"""

from __future__ import annotations

from .tree import Forest


def forest_stats(forest: Forest, seqs=None) -> dict:
    tree_tokens = sum(t.n_tokens for t in forest.trees)
    padded = sum(t.n_padded for t in forest.trees)
    orig = sum(t.orig_tokens for t in forest.trees)
    pairs = sum(t.n_pairs for t in forest.trees)
    causal = None
    if seqs is not None:
        causal = sum(len(s) * (len(s) + 1) // 2 for s in seqs)
    return dict(
        n_trees=len(forest.trees), tree_tokens=tree_tokens, padded_tokens=padded,
        orig_tokens=orig, tree_token_ratio=tree_tokens / orig,
        padded_ratio=padded / orig, pairs=pairs, causal_pairs=causal,
        n_tiles=sum(len(t.q_kb) for t in forest.trees),
    )


def attn_flops(pairs: int, hq: int, head_dim: int) -> dict:
    """Algorithmic FLOPs of tree attention over `pairs` visible (query, key)
    pairs per query head: forward 2 d for the score and 2 d for the P.V
    product per pair and head; backward 2.5 times that (dV, dP, dQ and dK
    products plus the recomputed scores).  fwd_bwd is their sum."""
    fwd = 4 * head_dim * hq * pairs
    return dict(fwd=fwd, bwd=2.5 * fwd, fwd_bwd=3.5 * fwd)
