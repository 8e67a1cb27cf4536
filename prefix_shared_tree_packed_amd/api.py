"""Thin Python binding of libpst.  Torch supplies device memory and streams;
every computation happens in the library.  Names follow the C ABI:

    build_tree(seqs, max_tokens_per_mb)            -> Forest       (host)
    tree_meta_create(forest, tree, stream=None)    -> TreeMeta     (device upload)
    forest_meta_create(forest, stream=None)        -> TreeMeta     (all trees back to back)
    TreeMeta.update(forest, stream=None)           -> re-upload into the same buffers
    tree_attn_fwd(q, k, v, meta, ...)              -> (o, lse)
    tree_attn_bwd(q, k, v, o, lse, dout, meta, ...) -> (dq, dk, dv)
    tree_attn_bwd_noalloc(q, k, v, o, lse, dout, meta, dq, dk, dv) -> (dq, dk, dv)
    gather_tree_logprobs_entropy(logits, meta, ...) -> (logprobs, entropy)
    gather_tree_logprobs_entropy_bwd(logits, meta, dlogprobs, dentropy) -> dlogits
    tree_rope(x, meta, theta=None, inverse=False)  -> x rotated in place
    tree_dense_mask(meta, format="u8")             -> [Np, Np] mask
    pack_allocate(values, capacity, ...)           -> (groups, fell_back)   (host)
    packing_metrics(values, groups, capacity)      -> dict                  (host)
    assign_trees(forest, n_ranks, ...)             -> rank of every tree    (host)
"""

from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_size_t, c_void_p
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import PST_BF16, PST_F32, PstError, check  # noqa: F401


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PST_BF16
    if t.dtype == torch.float32:
        return PST_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr_or_null(t):
    return 0 if t is None else t.data_ptr()


def _dev_tensor(t, name, dev=None):
    """A contiguous tensor on the current device (`dev`: its index, when the
    caller already has it; looked up once per call otherwise)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dev is None:
        import torch
        dev = torch.cuda.current_device()
    if t.get_device() != dev:
        raise ValueError(f"{name} is on cuda:{t.get_device()}, not the current device cuda:{dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _checked(t, name, shape, dtype, dev=None):
    """A caller-supplied buffer: a contiguous device tensor of exactly this
    shape and dtype (the library sees only its pointer, so a smaller or
    differently typed buffer would be read or written out of bounds)."""
    _dev_tensor(t, name, dev)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")
    return t


class Forest:
    """Sequences packed into compressed tries (host, library-owned)."""

    def __init__(self, seqs: Sequence, max_tokens_per_mb: int, pad_to_maximum: bool = False):
        lib = _lib.load()
        arrs = [np.ascontiguousarray(s, dtype=np.int32).ravel() for s in seqs]
        lens = np.array([a.size for a in arrs], dtype=np.int64)
        self._tokens = np.concatenate(arrs) if arrs else np.zeros(0, np.int32)
        self._offsets = np.zeros(len(arrs) + 1, dtype=np.int64)
        np.cumsum(lens, out=self._offsets[1:])
        self.n_seqs = len(arrs)
        h = c_void_p()
        self._h = None
        flags = _lib.PST_BUILD_PAD_TO_MAXIMUM if pad_to_maximum else 0
        check(lib.pst_build_tree_ex(
            self._tokens.ctypes.data_as(_lib.P32), self._offsets.ctypes.data_as(_lib.P64),
            int(self.n_seqs), int(max_tokens_per_mb), flags, byref(h)))
        self._h = h
        n = c_int32()
        check(lib.pst_forest_num_trees(self._h, byref(n)))
        self.n_trees = n.value

    def close(self):
        if self._h is not None:
            _lib.load().pst_forest_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sizes(self, tree: int) -> dict:
        s = _lib.TreeSizes()
        check(_lib.load().pst_forest_tree_sizes(self._h, int(tree), byref(s)))
        return {f: getattr(s, f) for f, _ in s._fields_}

    def stats(self) -> dict:
        s = _lib.Stats()
        check(_lib.load().pst_forest_stats(self._h, byref(s)))
        return {f: getattr(s, f) for f, _ in s._fields_}

    def seq_tree(self) -> np.ndarray:
        out = np.zeros(self.n_seqs, dtype=np.int32)
        check(_lib.load().pst_forest_seq_tree(self._h, out.ctypes.data_as(_lib.P32)))
        return out

    def export(self, tree: int) -> dict:
        """Every array of tree `tree` as numpy (see pst_tree_arrays)."""
        s = self.sizes(tree)
        shapes = {
            "token": s["n_padded"], "pos": s["n_padded"], "parent": s["n_padded"],
            "subtree_end": s["n_padded"], "node": s["n_padded"],
            "node_start": s["n_nodes"], "node_end": s["n_nodes"], "node_parent": s["n_nodes"],
            "node_seq_ptr": s["n_nodes"] + 1, "node_seq_ids": s["n_node_seq"],
            "seq_ids": s["n_seqs"], "seq_out_offsets": s["n_seqs"] + 1,
            "seq_index": s["n_out"], "child_ptr": s["n_tokens"] + 1, "child_idx": s["n_edges"],
            "q_ptr": s["n_blocks"] + 1, "q_kb": s["n_tiles"], "q_full": s["n_tiles"],
            "q_cls": s["n_tiles"],
            "kb_qhi": s["n_blocks"], "fwd_order": s["n_blocks"], "bwd_order": s["n_blocks"],
        }
        out, a = {}, _lib.TreeArrays()
        for name in _lib.ARRAY_FIELDS:
            dt = np.int64 if name == "seq_out_offsets" else np.int32
            arr = np.zeros(max(shapes[name], 0), dtype=dt)
            out[name] = arr
            setattr(a, name, arr.ctypes.data_as(_lib.P64 if dt == np.int64 else _lib.P32))
        check(_lib.load().pst_forest_export_tree(self._h, int(tree), byref(a)))
        return out


def build_tree(seqs: Sequence, max_tokens_per_mb: int, pad_to_maximum: bool = False) -> Forest:
    """Pack sequences into compressed tries; pad_to_maximum pads every tree to
    max_tokens_per_mb rows (fixed micro-batch shape)."""
    return Forest(seqs, max_tokens_per_mb, pad_to_maximum)


class TreeMeta:
    """Device-resident metadata of one tree (pst_tree_meta)."""

    def __init__(self, forest: Forest, tree: Optional[int], stream=None):
        """tree=None: the whole forest, trees back to back (pst_forest_meta_create)."""
        h = c_void_p()
        self._h = None
        lib = _lib.load()
        if tree is None:
            check(lib.pst_forest_meta_create(forest._h, c_void_p(_stream_ptr(stream)), byref(h)))
        else:
            check(lib.pst_tree_meta_create(forest._h, int(tree), c_void_p(_stream_ptr(stream)), byref(h)))
        self._h = h
        s = _lib.TreeSizes()
        check(_lib.load().pst_tree_meta_sizes(self._h, byref(s)))
        self.sizes = {f: getattr(s, f) for f, _ in s._fields_}
        self.n_padded = self.sizes["n_padded"]
        self.n_tokens = self.sizes["n_tokens"]
        self.n_out = self.sizes["n_out"]

    def update(self, forest: Forest, stream=None):
        """Re-upload for another forest (all its trees) into the same device
        and pinned buffers (pst_forest_meta_update): no allocation in steady
        state.  Work queued on `stream` that reads the old metadata runs
        first; work on other streams must have finished."""
        s = _lib.TreeSizes()
        lib = _lib.load()
        check(lib.pst_forest_meta_update(forest._h, c_void_p(_stream_ptr(stream)), self._h))
        check(lib.pst_tree_meta_sizes(self._h, byref(s)))
        self.sizes = {f: getattr(s, f) for f, _ in s._fields_}
        self.n_padded = self.sizes["n_padded"]
        self.n_tokens = self.sizes["n_tokens"]
        self.n_out = self.sizes["n_out"]
        return self

    def destroy(self):
        """Frees the device copy; the caller has synchronized every stream
        that used it."""
        if self._h is not None:
            check(_lib.load().pst_tree_meta_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            if self._h is not None:
                import torch
                torch.cuda.synchronize()
                self.destroy()
        except Exception:
            pass


def tree_meta_create(forest: Forest, tree: int, stream=None) -> TreeMeta:
    return TreeMeta(forest, tree, stream)


def forest_meta_create(forest: Forest, stream=None) -> TreeMeta:
    return TreeMeta(forest, None, stream)


def tree_attn_fwd(q, k, v, meta: TreeMeta, softmax_scale: Optional[float] = None,
                  out=None, lse=None, stream=None):
    import torch
    dev = torch.cuda.current_device()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, n, dev)
    Np, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (Np, hkv, d) or v.shape != k.shape or Np != meta.n_padded:
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)} "
                         f"do not match a tree of {meta.n_padded} padded rows")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    code = _dtype_code(q)
    out = torch.empty_like(q) if out is None else _checked(out, "out", q.shape, q.dtype, dev)
    lse = (torch.empty((hq, Np), dtype=torch.float32, device=q.device) if lse is None
           else _checked(lse, "lse", (hq, Np), torch.float32, dev))
    check(_lib.load().pst_tree_attn_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr(), meta._h, hq, hkv, d, code,
        float(softmax_scale or 0.0), c_void_p(_stream_ptr(stream))))
    return out, lse


def tree_attn_bwd_workspace_bytes(meta: TreeMeta, hq: int, hkv: int, head_dim: int,
                                  dtype: str) -> int:
    """Device workspace bytes of tree_attn_bwd for these shapes; dtype "f32" or "bf16"."""
    n = c_size_t()
    code = {"f32": 0, "bf16": 1}[dtype]
    check(_lib.load().pst_tree_attn_bwd_workspace_bytes(meta._h, hq, hkv, head_dim, code, byref(n)))
    return n.value


def _bwd_args(q, k, v, o, lse, dout, meta, dq, dk, dv):
    """Checked arguments of the backward entry points: (hq, hkv, d, dtype
    code, dq, dk, dv), outputs allocated when None."""
    import torch
    dev = torch.cuda.current_device()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (lse, "lse"), (dout, "dout")):
        _dev_tensor(t, n, dev)
    Np, hq, d = q.shape
    hkv = k.shape[1]
    if (k.shape != (Np, hkv, d) or v.shape != k.shape or o.shape != q.shape
            or dout.shape != q.shape or tuple(lse.shape) != (hq, Np) or Np != meta.n_padded):
        raise ValueError("shape mismatch in tree_attn_bwd arguments")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o, dout must share a dtype")
    if lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32, got {lse.dtype}")
    code = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else _checked(dq, "dq", q.shape, q.dtype, dev)
    dk = torch.empty_like(k) if dk is None else _checked(dk, "dk", k.shape, k.dtype, dev)
    dv = torch.empty_like(v) if dv is None else _checked(dv, "dv", v.shape, v.dtype, dev)
    return hq, hkv, d, code, dq, dk, dv


def tree_attn_bwd(q, k, v, o, lse, dout, meta: TreeMeta, softmax_scale: Optional[float] = None,
                  dq=None, dk=None, dv=None, workspace=None, stream=None):
    import torch
    hq, hkv, d, code, dq, dk, dv = _bwd_args(q, k, v, o, lse, dout, meta, dq, dk, dv)
    if workspace is None:
        nbytes = tree_attn_bwd_workspace_bytes(meta, hq, hkv, d,
                                               "bf16" if q.dtype == torch.bfloat16 else "f32")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _dev_tensor(workspace, "workspace", torch.cuda.current_device())
    check(_lib.load().pst_tree_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), meta._h, hq, hkv, d, code,
        float(softmax_scale or 0.0), c_void_p(_stream_ptr(stream))))
    return dq, dk, dv


def tree_attn_bwd_noalloc(q, k, v, o, lse, dout, meta: TreeMeta, dq, dk, dv,
                          softmax_scale: Optional[float] = None, stream=None):
    """tree_attn_bwd without a workspace: the library keeps the backward's
    scratch in a 64 MiB array of its own per GPU and allocates nothing
    (for code that cannot allocate, e.g. under graph capture).  The caller
    passes dq, dk, dv.  Calls that overlap in time on one GPU race."""
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is None:
            raise ValueError(f"{n} must be given: tree_attn_bwd_noalloc allocates nothing")
    hq, hkv, d, code, dq, dk, dv = _bwd_args(q, k, v, o, lse, dout, meta, dq, dk, dv)
    check(_lib.load().pst_tree_attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), meta._h, hq, hkv, d, code,
        float(softmax_scale or 0.0), c_void_p(_stream_ptr(stream))))
    return dq, dk, dv


def _row_stats(t, meta, name="row_stats", dev=None):
    import torch
    if t is None:
        return None
    return _checked(t, name, (meta.n_padded, 2), torch.float32, dev)


def gather_tree_logprobs_entropy(logits, meta: TreeMeta, logprobs=None, entropy=None,
                                 row_stats=None, stream=None):
    """Per-sequence logprobs and entropies.  row_stats (optional, float32
    [Np, 2]) receives (log-sum-exp, entropy) of every real row, which the
    backward can take instead of re-reading each row for them."""
    import torch
    dev = torch.cuda.current_device()
    _dev_tensor(logits, "logits", dev)
    if logits.dim() != 2 or logits.shape[0] != meta.n_padded:
        raise ValueError(f"logits must be [{meta.n_padded}, V], got {tuple(logits.shape)}")
    n = meta.n_out
    code = _dtype_code(logits)
    logprobs = (torch.empty(n, dtype=torch.float32, device=logits.device) if logprobs is None
                else _checked(logprobs, "logprobs", (n,), torch.float32, dev))
    entropy = (torch.empty(n, dtype=torch.float32, device=logits.device) if entropy is None
               else _checked(entropy, "entropy", (n,), torch.float32, dev))
    check(_lib.load().pst_gather_tree_logprobs_entropy(
        logits.data_ptr(), int(logits.shape[1]), code, meta._h,
        logprobs.data_ptr(), entropy.data_ptr(),
        c_void_p(_ptr_or_null(_row_stats(row_stats, meta, dev=dev))), c_void_p(_stream_ptr(stream))))
    return logprobs, entropy


def gather_tree_logprobs_entropy_bwd(logits, meta: TreeMeta, dlogprobs, dentropy, dlogits=None,
                                     row_stats=None, stream=None):
    """d logits of sum(dlogprobs * logprobs + dentropy * entropy); returns
    dlogits [Np, V] in the logits' dtype (pad rows zero).  row_stats: the
    forward gather's row statistics for these logits (optional)."""
    import torch
    dev = torch.cuda.current_device()
    _dev_tensor(logits, "logits", dev)
    if logits.dim() != 2 or logits.shape[0] != meta.n_padded:
        raise ValueError(f"logits must be [{meta.n_padded}, V], got {tuple(logits.shape)}")
    for t, name in ((dlogprobs, "dlogprobs"), (dentropy, "dentropy")):
        _checked(t, name, (meta.n_out,), torch.float32, dev)
    code = _dtype_code(logits)
    dlogits = (torch.empty_like(logits) if dlogits is None
               else _checked(dlogits, "dlogits", logits.shape, logits.dtype, dev))
    check(_lib.load().pst_gather_tree_logprobs_entropy_bwd(
        logits.data_ptr(), int(logits.shape[1]), code, meta._h,
        dlogprobs.data_ptr(), dentropy.data_ptr(),
        c_void_p(_ptr_or_null(_row_stats(row_stats, meta, dev=dev))),
        dlogits.data_ptr(), c_void_p(_stream_ptr(stream))))
    return dlogits


def tree_rope(x, meta: TreeMeta, theta: Optional[float] = None, inverse: bool = False, stream=None):
    """Rotary embedding of packed x [Np, heads, head_dim] in place with
    position = depth (inverse: the backward rotation); returns x."""
    _dev_tensor(x, "x")
    if x.dim() != 3 or x.shape[0] != meta.n_padded:
        raise ValueError(f"x must be [{meta.n_padded}, heads, head_dim], got {tuple(x.shape)}")
    check(_lib.load().pst_tree_rope(
        x.data_ptr(), meta._h, int(x.shape[1]), int(x.shape[2]), _dtype_code(x),
        float(theta or 0.0), int(bool(inverse)), c_void_p(_stream_ptr(stream))))
    return x


PACKING_ALGORITHMS = {"ffd": _lib.PST_PACK_FFD, "kk": _lib.PST_PACK_KK}


def pack_allocate(values, capacity: int, min_groups: int = 1, divisor: int = 1,
                  algorithm: str = "ffd"):
    """Allocate weighted items to groups with FFD or Karmarkar-Karp (host).
    Returns (groups, fell_back): groups is a list of item-index lists (items
    in ascending index), fell_back is True when KK fell back to FFD."""
    if algorithm not in PACKING_ALGORITHMS:
        raise ValueError(f"unknown packing algorithm {algorithm!r}; valid: "
                         + ", ".join(repr(a) for a in PACKING_ALGORITHMS))
    v = np.ascontiguousarray(values, dtype=np.int64).ravel()
    group_of = np.zeros(max(v.size, 1), dtype=np.int32)
    ng, fb = c_int32(), c_int32()
    check(_lib.load().pst_pack_allocate(
        v.ctypes.data_as(_lib.P64), v.size, int(capacity), int(min_groups), int(divisor),
        PACKING_ALGORITHMS[algorithm], group_of.ctypes.data_as(_lib.P32), byref(ng), byref(fb)))
    groups = [[] for _ in range(ng.value)]
    for i, g in enumerate(group_of[:v.size]):
        groups[int(g)].append(i)
    return groups, bool(fb.value)


def packing_metrics(values, groups, capacity: int) -> dict:
    """Spread, imbalance ratio, std_dev, cv, utilization and wasted tokens of
    an allocation (groups: lists of item indices covering every item)."""
    v = np.ascontiguousarray(values, dtype=np.int64).ravel()
    group_of = np.full(v.size, -1, dtype=np.int32)
    for g, items in enumerate(groups):
        group_of[list(items)] = g
    m = _lib.PackMetrics()
    check(_lib.load().pst_pack_metrics_compute(
        v.ctypes.data_as(_lib.P64), v.size, group_of.ctypes.data_as(_lib.P32), len(groups),
        int(capacity), byref(m)))
    return {f: getattr(m, f) for f, _ in m._fields_}


def assign_trees(forest: Forest, n_ranks: int, cost: str = "pairs", algorithm: str = "kk"):
    """Balance the trees of a forest over `n_ranks` data-parallel ranks with
    no capacity limit.  cost: "pairs" (visible attention pairs, the FLOP
    driver) or "tokens" (real tree tokens).  Returns the rank of every tree
    (int32 numpy array); with fewer trees than ranks some ranks get none."""
    key = {"pairs": "n_pairs", "tokens": "n_tokens"}.get(cost)
    if key is None:
        raise ValueError(f"unknown cost {cost!r}; valid: 'pairs', 'tokens'")
    n_trees = forest.stats()["n_trees"]
    costs = np.array([forest.sizes(t)[key] for t in range(n_trees)], dtype=np.int64)
    groups, _ = pack_allocate(costs, max(int(costs.sum()), 1), min_groups=n_ranks,
                              algorithm=algorithm)
    rank = np.zeros(n_trees, dtype=np.int32)
    for g, items in enumerate(groups):
        rank[items] = g
    return rank


MASK_FORMATS = {"u8": _lib.PST_MASK_U8, "add_f32": _lib.PST_MASK_ADD_F32,
                "add_bf16": _lib.PST_MASK_ADD_BF16}


def tree_dense_mask(meta: TreeMeta, format: str = "u8", out=None, stream=None):
    """Dense [Np, Np] attention mask of the tree(s) behind `meta` (row = query,
    column = key): "u8" (1 visible), "add_f32" / "add_bf16" (0 visible, -inf
    hidden).  Returns `out` (allocated when None)."""
    import torch
    if format not in MASK_FORMATS:
        raise ValueError(f"unknown mask format {format!r}; valid: {sorted(MASK_FORMATS)}")
    dt = {"u8": torch.uint8, "add_f32": torch.float32, "add_bf16": torch.bfloat16}[format]
    Np = meta.n_padded
    if out is None:
        out = torch.empty((Np, Np), dtype=dt, device="cuda")
    _dev_tensor(out, "out")
    if out.dtype != dt or tuple(out.shape) != (Np, Np):
        raise ValueError(f"out must be {dt} [{Np}, {Np}]")
    check(_lib.load().pst_tree_dense_mask(meta._h, MASK_FORMATS[format],
                                          c_void_p(out.data_ptr()), c_void_p(_stream_ptr(stream))))
    return out
