"""Oracle: rotary position embedding of packed tree tokens (test
infrastructure only).

The tree-training page's "Archon 引擎" section passes position_ids to the
model together with the tree metadata.  For a packed tree the position of a
token is the one it has in every sequence that contains it: its depth in the
trie, exported as `pos`.  So rotary embeddings of the packed Q and K use
pos = depth.  The rotation is the
standard one (RoFormer), in the rotate-half pairing: for head_dim d and
i < d/2, dims i and i + d/2 form a pair rotated by the angle
pos * theta^(-2i/d) (theta = 10000 unless given):

    y[i]       = x[i] cos(a) - x[i + d/2] sin(a)
    y[i + d/2] = x[i + d/2] cos(a) + x[i] sin(a)

The inverse (the rotation by -a) is the backward: the gradient of y with
respect to x applied to dy.  float64 throughout.
"""

from __future__ import annotations

import numpy as np


def rope(x, pos, theta: float = 10000.0, inverse: bool = False):
    """x: [rows, heads, d] (d even); pos: [rows] integer positions.
    Returns float64 [rows, heads, d]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half)) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    if inverse:
        ang = -ang
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
