"""The synthetic workloads of the tree-training hot path.

Each workload is a list of token sequences (sequences that share prefixes, as
produced by RL sampling), a packing capacity (tokens per tree, a multiple of
the 128-token block) and the attention/logit shapes that go with it.  The
shapes follow the five benchmark settings of this project:

  tiny      one 32-token prompt + 4 responses (8/16/24/32), two of which share
            their first 8 tokens; fp32, 2 heads, head_dim 64, vocab 256
  grpo      4 prompts x 512 tokens, 8 responses each, lengths U{128..1024};
            capacity 8192; bf16, 32 q heads / 8 kv heads, head_dim 128, vocab 32000
  agentic   2048-token system prompt, 16 trajectories of 4-8 turns
            (observation U{64..256} + action U{32..512}), each new trajectory
            forking at a turn boundary of an earlier one; capacity 16384;
            bf16 32/8, head_dim 128
  bimodal   64 prompts x 256 tokens x 4 samples, response lengths 70%
            U{50..200} and 30% U{800..2048}; capacity 8192; bf16 40/8,
            head_dim 128, vocab 152064
  long      2 prompts x 8192 tokens x 8 responses U{1024..4096}; capacity
            32768; bf16 64/8, head_dim 128
  long_control  the same 16 response lengths, each sequence with its own
            prompt (no sharing at all)

The bimodal length mix is the generator described on the micro-batch packing
page (AReaL seqpack article, section on the KK-vs-FFD experiment): short
responses 50-200 tokens, long ones 800-2048, 30% long.

Readings of what the settings leave open (all integers are drawn inclusive):
  * "two responses share their first 8 tokens" (tiny): responses 2 and 3.
  * Random ids can collide where sequences are meant to fork; at every
    intended fork the first new token is redrawn until it differs from the
    token at that position of every earlier sequence with the same prefix, so
    the intended sharing is exactly the sharing a trie finds.
  * agentic forks: parent e ~ U{0..k-1}, boundary b ~ U{0..n_e-1} (b = 0 is
    right after the system prompt), the new trajectory keeps the first b turns
    of e and then draws max(n_k - b, 1) fresh turns, n_k ~ U{4..8}.
  * Token ids of bimodal are drawn from its vocab [0,152064), of long from
    [0,32000).

Nothing here computes a trie, a mask or a softmax.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np


@dataclasses.dataclass
class Workload:
    name: str
    seqs: List[np.ndarray]          # int32 token arrays, in input order
    max_tokens_per_mb: int          # per-tree token capacity (multiple of 128)
    hq: int                         # query heads
    hkv: int                        # key/value heads
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    vocab: Optional[int]            # logit width of the gather, None if no gather
    fwd: bool = True
    bwd: bool = False
    gather: bool = False
    logit_std: float = 1.0
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        return int(sum(len(s) for s in self.seqs))


def _diverge(existing: List[np.ndarray], seq: np.ndarray, pos: int,
             rng: np.random.Generator, lo: int, hi: int) -> None:
    """Redraw seq[pos] until no earlier sequence with the same first `pos`
    tokens carries the same token at `pos` (in place)."""
    clash = [s for s in existing
             if len(s) > pos and np.array_equal(s[:pos], seq[:pos])]
    while any(int(s[pos]) == int(seq[pos]) for s in clash):
        seq[pos] = rng.integers(lo, hi)


def _tiny(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    vocab = 256
    prompt = rng.integers(0, vocab, size=32).astype(np.int32)
    seqs: List[np.ndarray] = []
    for r, L in enumerate((8, 16, 24, 32)):
        resp = rng.integers(0, vocab, size=L).astype(np.int32)
        s = np.concatenate([prompt, resp])
        if r == 3:
            # responses 2 and 3 share their first 8 tokens
            s[32:40] = seqs[2][32:40]
            _diverge(seqs, s, 40, rng, 0, vocab)
        else:
            _diverge(seqs, s, 32, rng, 0, vocab)
        seqs.append(s)
    return Workload("tiny", seqs, 128, hq=2, hkv=2, head_dim=64, dtype="f32",
                    vocab=vocab, fwd=True, bwd=False, gather=True,
                    logit_std=1.0, seed=seed)


def _prompt_groups(rng, n_prompts, prompt_len, n_resp, len_fn, vocab):
    seqs: List[np.ndarray] = []
    for _p in range(n_prompts):
        prompt = rng.integers(0, vocab, size=prompt_len).astype(np.int32)
        first_of_group = len(seqs)
        for r in range(n_resp):
            L = int(len_fn(rng))
            resp = rng.integers(0, vocab, size=L).astype(np.int32)
            s = np.concatenate([prompt, resp])
            if r == 0:
                _diverge(seqs, s, 0, rng, 0, vocab)
                prompt = s[:prompt_len].copy()
            else:
                _diverge(seqs[first_of_group:], s, prompt_len, rng, 0, vocab)
            seqs.append(s)
    return seqs


def _grpo(seed: int = 2) -> Workload:
    rng = np.random.default_rng(seed)
    seqs = _prompt_groups(rng, 4, 512, 8, lambda g: g.integers(128, 1025), 32000)
    return Workload("grpo", seqs, 8192, hq=32, hkv=8, head_dim=128, dtype="bf16",
                    vocab=32000, fwd=True, bwd=False, gather=True,
                    logit_std=2.0, seed=seed)


def _agentic(seed: int = 3) -> Workload:
    rng = np.random.default_rng(seed)
    vocab = 32000
    system = rng.integers(0, vocab, size=2048).astype(np.int32)
    turns: List[List[np.ndarray]] = []      # per trajectory, its turns
    seqs: List[np.ndarray] = []

    def fresh_turn():
        obs = rng.integers(0, vocab, size=int(rng.integers(64, 257)))
        act = rng.integers(0, vocab, size=int(rng.integers(32, 513)))
        return np.concatenate([obs, act]).astype(np.int32)

    for k in range(16):
        n_k = int(rng.integers(4, 9))
        if k == 0:
            b, kept = 0, []
        else:
            e = int(rng.integers(0, k))
            b = int(rng.integers(0, len(turns[e])))
            kept = turns[e][:b]
        new = [fresh_turn() for _ in range(max(n_k - b, 1))]
        s = np.concatenate([system] + kept + new).astype(np.int32)
        fork = len(system) + sum(len(t) for t in kept)
        if k > 0:
            _diverge(seqs, s, fork, rng, 0, vocab)
            # the redraw may have changed the first token of the first fresh turn
            new[0] = s[fork:fork + len(new[0])].copy()
        turns.append(kept + new)
        seqs.append(s)
    return Workload("agentic", seqs, 16384, hq=32, hkv=8, head_dim=128,
                    dtype="bf16", vocab=None, fwd=True, bwd=True, gather=False,
                    seed=seed)


def _bimodal(seed: int = 4) -> Workload:
    rng = np.random.default_rng(seed)

    def length(g):
        if g.random() < 0.3:
            return g.integers(800, 2049)
        return g.integers(50, 201)

    seqs = _prompt_groups(rng, 64, 256, 4, length, 152064)
    return Workload("bimodal", seqs, 8192, hq=40, hkv=8, head_dim=128,
                    dtype="bf16", vocab=152064, fwd=True, bwd=True, gather=True,
                    logit_std=2.0, seed=seed)


def _long(seed: int = 5) -> Workload:
    rng = np.random.default_rng(seed)
    seqs = _prompt_groups(rng, 2, 8192, 8, lambda g: g.integers(1024, 4097), 32000)
    return Workload("long", seqs, 32768, hq=64, hkv=8, head_dim=128, dtype="bf16",
                    vocab=None, fwd=True, bwd=True, gather=False, seed=seed)


def _long_control(seed: int = 55) -> Workload:
    """Same 16 response lengths as `long`, every sequence with its own prompt."""
    lengths = [len(s) - 8192 for s in _long().seqs]
    rng = np.random.default_rng(seed)
    seqs: List[np.ndarray] = []
    for L in lengths:
        s = rng.integers(0, 32000, size=8192 + L).astype(np.int32)
        _diverge(seqs, s, 0, rng, 0, 32000)
        seqs.append(s)
    return Workload("long_control", seqs, 32768, hq=64, hkv=8, head_dim=128,
                    dtype="bf16", vocab=None, fwd=True, bwd=True, gather=False,
                    seed=seed)


WORKLOADS = {
    "tiny": _tiny,
    "grpo": _grpo,
    "agentic": _agentic,
    "bimodal": _bimodal,
    "long": _long,
    "long_control": _long_control,
}


def bimodal_lengths(n: int, seed: int) -> np.ndarray:
    """Sequence lengths of the packing page's bimodal generator: 70 %
    U{50..200}, 30 % U{800..2048} (int64 [n])."""
    rng = np.random.default_rng(seed)
    long = rng.random(n) < 0.3
    return np.where(long, rng.integers(800, 2049, size=n), rng.integers(50, 201, size=n)).astype(np.int64)


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]()
    except KeyError:
        raise ValueError(f"unknown workload {name!r}; choose from {sorted(WORKLOADS)}")


def worked_example() -> List[np.ndarray]:
    """The three sequences of the tree-construction figure on the tree
    training page (section "树构建过程"): ABCD, ABEF, AGH, with A..H = 1..8."""
    A, B, C, D, E, F, G, H = range(1, 9)
    return [np.array(x, dtype=np.int32) for x in
            ([A, B, C, D], [A, B, E, F], [A, G, H])]


def worked_example_edge() -> List[np.ndarray]:
    """The worked example plus a fourth sequence AG that ends inside the
    G-H chain."""
    return worked_example() + [np.array([1, 7], dtype=np.int32)]


def tree_tensor_seed(workload_seed: int, tree: int, name: str) -> int:
    """A stable 63-bit seed for tensor `name` of tree `tree`."""
    h = hashlib.sha256(f"{workload_seed}/{tree}/{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def make_tensor(shape, dtype: str, seed: int, device="cpu", std: float = 1.0):
    """i.i.d. N(0, std^2) values, drawn in fp32 from a seeded torch generator on
    `device`, then rounded to `dtype` ("f32" or "bf16", round to nearest even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return t
