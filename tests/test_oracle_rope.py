"""Pins of the oracle's tree-position rotary embedding (CPU only).

 * the same rotation written with complex numbers: (x_i + j x_{i+d/2}) times
   exp(j pos theta^(-2i/d));
 * position 0 is the identity; every (i, i + d/2) pair keeps its norm; the
   inverse undoes the forward;
 * scores depend only on relative position: <R(m) q, R(n) k> is unchanged
   when m and n move together;
 * on a packed tree (pos = depth) every token's result equals the rotary
   embedding of each sequence through it at positions 0 .. L-1, read
   through the sequence's index map.
"""

import numpy as np

import oracle
from workloads import worked_example


def test_complex_form():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 3, 16))
    pos = rng.integers(0, 5000, size=7)
    y = oracle.rope(x, pos, theta=500.0)
    half = 8
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(
        1j * pos[:, None, None] * 500.0 ** (-(2.0 * np.arange(half)) / 16))
    assert np.abs(y[..., :half] - z.real).max() < 1e-12
    assert np.abs(y[..., half:] - z.imag).max() < 1e-12


def test_identity_norms_inverse():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(9, 2, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(9, int)), x)
    pos = rng.integers(0, 32768, size=9)
    y = oracle.rope(x, pos)
    n_x = x[..., :32] ** 2 + x[..., 32:] ** 2
    n_y = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.abs(n_x - n_y).max() < 1e-10
    assert np.abs(oracle.rope(y, pos, inverse=True) - x).max() < 1e-10


def test_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=(1, 1, 128)), rng.normal(size=(1, 1, 128))
    dots = []
    for shift in (0, 17, 3000):
        rq = oracle.rope(q, np.array([40 + shift]))
        rk = oracle.rope(k, np.array([11 + shift]))
        dots.append(float((rq * rk).sum()))
    assert max(dots) - min(dots) < 1e-9


def test_packed_equals_per_sequence():
    rng = np.random.default_rng(3)
    seqs = worked_example() + [np.array([1, 2, 3, 4, 9, 9], np.int32)]
    tree = oracle.build_forest(seqs, 128).trees[0]
    x = rng.normal(size=(tree.n_padded, 2, 32))
    y = oracle.rope(x, tree.pos)
    for sid in tree.seq_ids:
        idx = tree.seq_index[sid]
        ys = oracle.rope(x[idx], np.arange(len(idx)))
        assert np.abs(y[idx] - ys).max() < 1e-12
