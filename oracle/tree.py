"""Oracle: packing sequences into compressed tries (test infrastructure only).

Follows the four construction steps of the AReaL tree-training page (section
"树构建过程"): take each sequence's real tokens, insert sequences greedily into
tries first-fit-decreasing, merge linear chains into single nodes, and derive
the block structure used by attention.  Node fields follow the TrieNode
dataclass of the same page (section "数据结构 / TrieNode").  The capacity is the
maximum number of tokens per tree and must be a multiple of the 128-token
block (section "必需配置").

Readings of points the page leaves open (each the plainest one):
  * first fit: a sequence goes into the first tree, in creation order, whose
    token count after sharing stays within the capacity; otherwise it opens a
    new tree;
  * "decreasing" is by sequence length, ties broken by input index;
  * children keep first-insertion order, which is also preorder order;
  * a node also ends after any token where a sequence ends, so every sequence
    is a union of whole nodes;
  * the root is virtual (start = end = -1); depth-0 tokens have parent -1;
  * the flattened tree is padded to the next multiple of 128 with pad tokens
    (id 0, position 0, parent -1) that see only themselves;
  * pad_to_maximum (configuration section, 启用树训练): every tree is padded
    to the capacity itself instead, with the same pad tokens.

Everything below is written for clarity: dictionaries for the trie, explicit
walks of parent chains for the ancestor relation, brute-force scans for the
tile classes.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

BLOCK = 128  # BLOCK_SIZE of the tree-training page (section "带块掩码的 FlexAttention")


class OracleError(ValueError):
    code = "EINVAL"


class InvalidInput(OracleError):
    code = "EINVAL"


class CapacityError(OracleError):
    code = "ECAPACITY"


class BlockError(OracleError):
    code = "EBLOCK"


class _TrieTok:
    """One token of the uncompressed trie."""
    __slots__ = ("token", "children", "parent", "passing", "ending", "flat")

    def __init__(self, token, parent):
        self.token = token
        self.children: Dict[int, "_TrieTok"] = {}   # insertion ordered
        self.parent = parent
        self.passing: List[int] = []   # ids of sequences through this token
        self.ending: List[int] = []    # ids of sequences whose last token this is
        self.flat = -1


@dataclasses.dataclass
class Node:
    """A compressed trie node (the page's TrieNode).  `children` maps the first
    token of each child to that child's index in `Tree.nodes`; `ancestors`
    lists node indices from the root down, the virtual root written as -1."""
    tree_id: int
    start_idx: int
    end_idx: int               # inclusive
    tokens: List[int]
    sequence_ids: List[int]
    children: Dict[int, int]
    ancestors: List[int]
    parent: int                # index of the parent node, -1 for the root


@dataclasses.dataclass
class Tree:
    tree_id: int
    n_tokens: int              # N, real tree tokens
    n_padded: int              # Np
    token: np.ndarray          # [Np] int32
    pos: np.ndarray            # [Np] int32 depth (index inside every sequence through it)
    parent: np.ndarray         # [Np] int32 flat index of the parent token, -1 at depth 0 / pads
    subtree_end: np.ndarray    # [Np] int32 last flat index of the token's subtree
    node: np.ndarray           # [Np] int32 compressed node of each token, -1 for pads
    root: Node                 # virtual root (start = end = -1)
    nodes: List[Node]          # compressed nodes in preorder
    seq_ids: List[int]         # input indices of the sequences in this tree, ascending
    seq_index: Dict[int, np.ndarray]   # input index -> flat index of each of its tokens
    out_offsets: np.ndarray    # [n_seqs+1] int64 offsets of each sequence's outputs
    child_ptr: np.ndarray      # [N+1] int32
    child_idx: np.ndarray      # [n_edges] int32 flat index of each child token
    q_ptr: np.ndarray          # [nb+1] int32, non-empty tiles of each query block
    q_kb: np.ndarray           # [n_tiles] int32 key block, descending within a query block
    q_full: np.ndarray         # [n_tiles] int32 1 if every pair of the tile is visible
    q_cls: np.ndarray          # [n_tiles] int32: 2 bits per 32x32 sub-block (query
                               #   sub-block qs, key sub-block ks) at bit 2*(4*qs+ks):
                               #   0 no visible pair, 1 some, 2 all
    kb_qhi: np.ndarray         # [nb] int32 last query block that sees the key block
    fwd_order: np.ndarray      # [nb] query blocks by tile count desc, then index
    bwd_order: np.ndarray      # [nb] key blocks by tile count desc, then index
    n_pairs: int               # visible (query, key) pairs among real tokens
    orig_tokens: int           # sum of the lengths of the tree's sequences

    @property
    def n_blocks(self) -> int:
        return self.n_padded // BLOCK


@dataclasses.dataclass
class Forest:
    trees: List[Tree]
    n_seqs: int
    max_tokens_per_mb: int
    seq_tree: np.ndarray       # [n_seqs] tree of each input sequence


def _validate(seqs, cap):
    if not isinstance(cap, (int, np.integer)) or cap <= 0:
        raise InvalidInput(f"max_tokens_per_mb must be positive, got {cap}")
    if cap % BLOCK:
        raise BlockError(f"max_tokens_per_mb={cap} is not a multiple of {BLOCK}")
    if len(seqs) == 0:
        raise InvalidInput("no sequences")
    for i, s in enumerate(seqs):
        if len(s) == 0:
            raise InvalidInput(f"sequence {i} is empty")
        if len(s) > cap:
            raise CapacityError(f"sequence {i} has {len(s)} tokens > max_tokens_per_mb={cap}")


def _shared_prefix(root: _TrieTok, seq) -> int:
    """Number of leading tokens of `seq` already present in the trie."""
    n, cur = 0, root
    for t in seq:
        nxt = cur.children.get(int(t))
        if nxt is None:
            break
        cur, n = nxt, n + 1
    return n


def _insert(root: _TrieTok, sid: int, seq) -> None:
    cur = root
    cur.passing.append(sid)
    for t in seq:
        t = int(t)
        nxt = cur.children.get(t)
        if nxt is None:
            nxt = _TrieTok(t, cur)
            cur.children[t] = nxt
        cur = nxt
        cur.passing.append(sid)
    cur.ending.append(sid)


def _preorder(root: _TrieTok) -> List[_TrieTok]:
    out, stack = [], list(reversed(list(root.children.values())))
    while stack:
        t = stack.pop()
        out.append(t)
        stack.extend(reversed(list(t.children.values())))
    return out


def build_forest(seqs, max_tokens_per_mb: int, pad_to_maximum: bool = False) -> Forest:
    """Pack `seqs` (sequences of token ids) into compressed, flattened, padded
    tries of at most `max_tokens_per_mb` tokens each.  With pad_to_maximum
    every tree is padded to max_tokens_per_mb rows."""
    seqs = [np.asarray(s, dtype=np.int64) for s in seqs]
    cap = max_tokens_per_mb
    _validate(seqs, cap)

    # step 2: first-fit decreasing insertion
    order = sorted(range(len(seqs)), key=lambda s: (-len(seqs[s]), s))
    tries: List[_TrieTok] = []
    counts: List[int] = []
    members: List[List[int]] = []
    for sid in order:
        seq = seqs[sid]
        for t, root in enumerate(tries):
            cost = len(seq) - _shared_prefix(root, seq)
            if counts[t] + cost <= cap:
                _insert(root, sid, seq)
                counts[t] += cost
                members[t].append(sid)
                break
        else:
            root = _TrieTok(-1, None)
            _insert(root, sid, seq)
            tries.append(root)
            counts.append(len(seq))
            members.append([sid])

    seq_tree = np.full(len(seqs), -1, dtype=np.int32)
    trees = []
    for tid, root in enumerate(tries):
        trees.append(_flatten(tid, root, seqs, sorted(members[tid]),
                              cap if pad_to_maximum else None))
        for sid in members[tid]:
            seq_tree[sid] = tid
    return Forest(trees, len(seqs), cap, seq_tree)


def _flatten(tid: int, root: _TrieTok, seqs, seq_ids: List[int], pad_to=None) -> Tree:
    toks = _preorder(root)
    N = len(toks)
    for i, t in enumerate(toks):
        t.flat = i
    Np = -(-N // BLOCK) * BLOCK if pad_to is None else pad_to

    token = np.zeros(Np, np.int32)
    pos = np.zeros(Np, np.int32)
    parent = np.full(Np, -1, np.int32)
    for i, t in enumerate(toks):      # preorder: a parent precedes its children
        token[i] = t.token
        if t.parent is not root:
            parent[i] = t.parent.flat
            pos[i] = pos[parent[i]] + 1

    # step 3: chain compression.  A token closes its node when it does not have
    # exactly one child or when some sequence ends on it.
    node = np.full(Np, -1, np.int32)
    root_node = Node(tid, -1, -1, [], sorted(root.passing), {}, [], -1)
    nodes: List[Node] = []
    opener = {}   # first token of a node -> node index
    for i, t in enumerate(toks):
        starts = t.parent is root or len(t.parent.children) != 1 or t.parent.ending
        if starts:
            if t.parent is root:
                par, anc = -1, [-1]
            else:
                par = node[t.parent.flat]
                anc = nodes[par].ancestors + [par]
            nodes.append(Node(tid, i, i, [t.token], sorted(t.passing), {}, anc, par))
            k = len(nodes) - 1
            opener[i] = k
            if par == -1:
                root_node.children[t.token] = k
            else:
                nodes[par].children[t.token] = k
        else:
            k = node[t.parent.flat]
            nodes[k].end_idx = i
            nodes[k].tokens.append(t.token)
        node[i] = k

    subtree_end, tiles = _walk_ancestors(N, Np, parent)

    # sequence maps: walk the trie along each sequence
    seq_index = {}
    offsets = [0]
    for sid in seq_ids:
        cur, idx = root, []
        for tkn in seqs[sid]:
            cur = cur.children[int(tkn)]
            idx.append(cur.flat)
        seq_index[sid] = np.array(idx, dtype=np.int32)
        offsets.append(offsets[-1] + len(idx))

    # child targets: distinct next tokens of every real token
    child_ptr = [0]
    child_idx: List[int] = []
    for t in toks:
        child_idx.extend(c.flat for c in t.children.values())
        child_ptr.append(len(child_idx))

    return Tree(
        tree_id=tid, n_tokens=N, n_padded=Np, token=token, pos=pos, parent=parent,
        subtree_end=subtree_end, node=node, root=root_node, nodes=nodes,
        seq_ids=list(seq_ids), seq_index=seq_index,
        out_offsets=np.array(offsets, dtype=np.int64),
        child_ptr=np.array(child_ptr, dtype=np.int32),
        child_idx=np.array(child_idx, dtype=np.int32),
        orig_tokens=int(sum(len(seqs[s]) for s in seq_ids)),
        **tiles,
    )


def _walk_ancestors(N: int, Np: int, parent: np.ndarray):
    """Enumerate every visible (query, key) pair straight from the ancestor
    relation -- query i sees itself and every token on its parent chain; a pad
    query sees only itself -- one ancestor level at a time for all queries.

    From the pairs: subtree_end[j] is the largest query that sees key j, and
    each 128x128 block of the mask is classified by how many of its pairs are
    visible (none: empty, all: full, else partial)."""
    nb = Np // BLOCK
    n32 = Np // 32
    subtree_end = np.arange(Np, dtype=np.int32)
    count32 = np.zeros(n32 * n32, dtype=np.int64)   # visible pairs per 32x32 block
    q = np.arange(N, dtype=np.int32)
    cur = q.copy()
    n_pairs = 0
    pending, n_pending = [], 0

    def flush():
        nonlocal count32, pending, n_pending
        if pending:
            ids = np.concatenate(pending)
            count32 += np.bincount(ids, minlength=n32 * n32)
        pending, n_pending = [], 0

    while q.size:
        np.maximum.at(subtree_end, cur, q)
        pending.append((q >> 5).astype(np.int64) * n32 + (cur >> 5))
        n_pending += q.size
        if n_pending > (1 << 25):
            flush()
        n_pairs += q.size
        nxt = parent[cur]
        keep = nxt >= 0
        q, cur = q[keep], nxt[keep]
    flush()
    pads = np.arange(N, Np, dtype=np.int64)
    count32 += np.bincount((pads >> 5) * n32 + (pads >> 5), minlength=n32 * n32)
    count32 = count32.reshape(n32, n32)              # [query sub-block, key sub-block]
    count = count32.reshape(nb, 4, nb, 4).sum(axis=(1, 3))   # [query block, key block]

    q_ptr, q_kb, q_full, q_cls = [0], [], [], []
    for qb in range(nb):
        for kb in range(nb - 1, -1, -1):
            if count[qb, kb] > 0:
                q_kb.append(kb)
                q_full.append(1 if count[qb, kb] == BLOCK * BLOCK else 0)
                bits = 0
                for qs in range(4):
                    for ks in range(4):
                        n = count32[4 * qb + qs, 4 * kb + ks]
                        cls = 0 if n == 0 else (2 if n == 32 * 32 else 1)
                        bits |= cls << (2 * (4 * qs + ks))
                q_cls.append(bits)
        q_ptr.append(len(q_kb))
    kb_qhi = np.array([max(qb for qb in range(nb) if count[qb, kb] > 0)
                       for kb in range(nb)], dtype=np.int32)
    per_q = (count > 0).sum(axis=1)
    per_k = (count > 0).sum(axis=0)
    fwd_order = sorted(range(nb), key=lambda b: (-per_q[b], b))
    bwd_order = sorted(range(nb), key=lambda b: (-per_k[b], b))
    return subtree_end.astype(np.int32), dict(
        q_ptr=np.array(q_ptr, np.int32), q_kb=np.array(q_kb, np.int32),
        q_full=np.array(q_full, np.int32), kb_qhi=kb_qhi,
        q_cls=np.array(q_cls, np.uint32).view(np.int32),
        fwd_order=np.array(fwd_order, np.int32),
        bwd_order=np.array(bwd_order, np.int32), n_pairs=int(n_pairs),
    )
