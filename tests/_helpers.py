"""Shared helpers of the GPU parity tests: build a case with both the library
and the oracle, draw seeded inputs on the device, compare with tolerances.

Tolerances (float outputs; integer outputs are compared bit-exactly):
  fp32 attention O, LSE:  |got - ref| <= 1e-5 |ref| + 1e-6
  bf16 attention O, LSE:  |got - ref| <= 2e-2
  fp32 gradients:         |got - ref| <= 1e-5 mag, entry by entry
  bf16 gradients:         |got - ref| <= 2e-2 + 2^-8 |ref|, or, where a test
                          passes the term magnitudes, <= 2^-6 mag entry by entry
  logprob/entropy:        |got - ref| <= 1e-3 from bf16 logits, 1e-5 |ref| + 1e-6 from fp32

mag is the entry's own sum of the sizes of the products it is built from
(oracle.attn_bwd_magnitudes: s sum_j P_ij (A_ij + B_i) |K_j| for dQ, with
A_ij = |dO_i|.|V_j| and B_i = |dO_i|.(sum_j P_ij |V_j|) the absolute sums
behind dP_ij and D_i, and so on): a float32 result whose products are each
rounded to a few units of 2^-24 is off by at most a small multiple of
2^-24 mag, and mag >= |ref|.  The bound is local to the entry: dS = P (dP - D)
cancels where dP and D agree (a token that sees only itself has dP = D
exactly, so its exact dQ and dK are 0), and the dot products inside dP and D
can cancel as well; there the computed value is rounding of the products,
which only their sizes bound.
A bf16 gradient is rounded once on output (half an ulp, at most 2^-8 of its
magnitude) on top of the bf16 rounding of P in its products; heavily shared
prefix tokens reach |dV| of several units, where the output rounding alone
exceeds 2e-2.  Where the gradients are large and cancel (a peaked softmax,
dP - D small on the dominant keys), the rounding of the bf16 O that D is
formed from reaches them too; every term passes through at most four bf16
roundings (O, P, dS, the output), hence 4 * 2^-8 mag.
"""

from __future__ import annotations

import numpy as np

import oracle
import prefix_shared_tree_packed_amd as pst
from workloads import make_tensor, tree_tensor_seed


def tol(dtype):
    return (1e-5, 1e-6) if dtype == "f32" else (0.0, 2e-2)


def assert_close(got, ref, dtype, what, rtol=None, atol=None, grad=False, mag=None):
    r, a = tol(dtype)
    r = r if rtol is None else rtol
    a = a if atol is None else atol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    if grad and dtype == "f32":
        assert mag is not None, "fp32 gradients are bounded by their term magnitudes"
        bound = 1e-5 * np.asarray(mag, dtype=np.float64)
    elif grad and mag is not None:
        # bf16 against the term magnitudes: every term of a gradient entry
        # passes through four bf16 roundings (O, which D is formed from; P;
        # dS; the output), each at most 2^-8 of its size
        bound = 2.0 ** -6 * np.asarray(mag, dtype=np.float64)
    elif grad:
        bound = 2e-2 + 2.0 ** -8 * np.abs(ref)
    else:
        bound = a + r * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{err.size} out of tolerance; worst at {idx}: "
            f"got {got[idx]!r} ref {ref[idx]!r} (max abs err {err.max():.3g})")


def torch_dtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def host(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def host32(t):
    """float32 host copy (exact for bf16 and fp32 values; half the memory of
    float64 for the full-size sampled checks)."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def attn_inputs(Np, hq, hkv, d, dtype, seed, device="cuda", with_dout=False):
    q = make_tensor((Np, hq, d), dtype, tree_tensor_seed(seed, 0, "q"), device)
    k = make_tensor((Np, hkv, d), dtype, tree_tensor_seed(seed, 0, "k"), device)
    v = make_tensor((Np, hkv, d), dtype, tree_tensor_seed(seed, 0, "v"), device)
    if not with_dout:
        return q, k, v
    do = make_tensor((Np, hq, d), dtype, tree_tensor_seed(seed, 0, "do"), device)
    return q, k, v, do


class Case:
    """One forest built twice: by the library (device metadata) and by the oracle."""

    def __init__(self, seqs, cap, pad_to_maximum=False):
        self.seqs = seqs
        self.forest = pst.build_tree(seqs, cap, pad_to_maximum=pad_to_maximum)
        self.ref = oracle.build_forest(seqs, cap, pad_to_maximum=pad_to_maximum)
        assert self.forest.n_trees == len(self.ref.trees)
        self.metas = [pst.tree_meta_create(self.forest, t) for t in range(self.forest.n_trees)]

    def close(self):
        import torch
        torch.cuda.synchronize()
        for m in self.metas:
            m.destroy()
        self.forest.close()


def prompt_groups(rng, n_prompts, prompt_len, n_resp, resp_lo, resp_hi, vocab=1000):
    seqs = []
    for p in range(n_prompts):
        prompt = rng.integers(0, vocab, size=prompt_len)
        prompt[0] = p  # distinct roots
        for r in range(n_resp):
            resp = rng.integers(0, vocab, size=int(rng.integers(resp_lo, resp_hi + 1)))
            resp[0] = r  # distinct forks
            seqs.append(np.concatenate([prompt, resp]).astype(np.int32))
    return seqs
