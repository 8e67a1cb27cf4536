"""ctypes declarations of libpst's C ABI (include/pst.h).  Argument marshalling
only; every step of the path runs inside the library."""

from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
# PST_LIBRARY selects another build of the library (the CPU sanitizer build of
# the host entry points, for instance); by default the in-tree libpst.so
LIB_PATH = os.environ.get("PST_LIBRARY") or os.path.join(PKG, "libpst.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pst.h")

PST_OK = 0
ERRORS = {
    -1: "PST_EINVAL", -2: "PST_ECAPACITY", -3: "PST_EBLOCK", -4: "PST_EDTYPE",
    -5: "PST_ESHAPE", -6: "PST_EHIP", -7: "PST_ENOMEM", -8: "PST_ERANGE",
}
PST_F32, PST_BF16 = 0, 1


class TreeSizes(ctypes.Structure):
    _fields_ = [
        ("n_tokens", c_int32), ("n_padded", c_int32), ("n_blocks", c_int32),
        ("n_nodes", c_int32), ("n_seqs", c_int32), ("n_edges", c_int32),
        ("n_tiles", c_int32), ("n_node_seq", c_int32), ("n_out", c_int64),
        ("n_pairs", c_int64),
    ]


P32 = POINTER(c_int32)
P64 = POINTER(c_int64)

ARRAY_FIELDS = [
    "token", "pos", "parent", "subtree_end", "node", "node_start", "node_end",
    "node_parent", "node_seq_ptr", "node_seq_ids", "seq_ids", "seq_out_offsets",
    "seq_index", "child_ptr", "child_idx", "q_ptr", "q_kb", "q_full", "q_cls", "kb_qhi",
    "fwd_order", "bwd_order",
]


class TreeArrays(ctypes.Structure):
    _fields_ = [(n, P64 if n == "seq_out_offsets" else P32) for n in ARRAY_FIELDS]


class Stats(ctypes.Structure):
    _fields_ = [
        ("n_trees", c_int32), ("n_seqs", c_int32), ("orig_tokens", c_int64),
        ("tree_tokens", c_int64), ("padded_tokens", c_int64), ("n_pairs", c_int64),
        ("causal_pairs", c_int64), ("n_tiles", c_int64), ("tree_token_ratio", c_double),
    ]


PST_PACK_FFD, PST_PACK_KK = 0, 1
PST_BUILD_PAD_TO_MAXIMUM = 1
PST_MASK_U8, PST_MASK_ADD_F32, PST_MASK_ADD_BF16 = 0, 1, 2


class PackMetrics(ctypes.Structure):
    _fields_ = [
        ("n_groups", c_int32), ("total", c_int64), ("max_load", c_int64),
        ("min_load", c_int64), ("spread", c_int64), ("wasted_tokens", c_int64),
        ("imbalance_ratio", c_double), ("std_dev", c_double), ("cv", c_double),
        ("utilization", c_double),
    ]


_SIGS = {
    "pst_build_tree": (c_int32, [P32, P64, c_int32, c_int32, POINTER(c_void_p)]),
    "pst_forest_num_trees": (c_int32, [c_void_p, P32]),
    "pst_forest_tree_sizes": (c_int32, [c_void_p, c_int32, POINTER(TreeSizes)]),
    "pst_forest_export_tree": (c_int32, [c_void_p, c_int32, POINTER(TreeArrays)]),
    "pst_forest_seq_tree": (c_int32, [c_void_p, P32]),
    "pst_forest_stats": (c_int32, [c_void_p, POINTER(Stats)]),
    "pst_forest_free": (None, [c_void_p]),
    "pst_tree_meta_create": (c_int32, [c_void_p, c_int32, c_void_p, POINTER(c_void_p)]),
    "pst_forest_meta_create": (c_int32, [c_void_p, c_void_p, POINTER(c_void_p)]),
    "pst_tree_meta_sizes": (c_int32, [c_void_p, POINTER(TreeSizes)]),
    "pst_forest_meta_update": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "pst_tree_meta_destroy": (c_int32, [c_void_p]),
    "pst_tree_attn_fwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int32, c_int32, c_int32, c_int32, c_float, c_void_p]),
    "pst_tree_attn_bwd_workspace_bytes": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32,
                                                     POINTER(c_size_t)]),
    "pst_tree_attn_bwd": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                    c_int32, c_int32, c_int32, c_int32, c_float, c_void_p]),
    "pst_tree_attn_bwd_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_int32, c_int32, c_int32, c_int32, c_float,
                                            c_void_p]),
    "pst_gather_tree_logprobs_entropy": (c_int32, [c_void_p, c_int64, c_int32, c_void_p,
                                                   c_void_p, c_void_p, c_void_p, c_void_p]),
    "pst_gather_tree_logprobs_entropy_bwd": (c_int32, [c_void_p, c_int64, c_int32, c_void_p,
                                                       c_void_p, c_void_p, c_void_p, c_void_p,
                                                       c_void_p]),
    "pst_tree_rope": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float, c_int32,
                                c_void_p]),
    "pst_pack_allocate": (c_int32, [P64, c_int32, c_int64, c_int32, c_int32, c_int32, P32, P32,
                                    P32]),
    "pst_pack_metrics_compute": (c_int32, [P64, c_int32, P32, c_int32, c_int64,
                                           POINTER(PackMetrics)]),
    "pst_build_tree_ex": (c_int32, [P32, P64, c_int32, c_int32, c_int32, POINTER(c_void_p)]),
    "pst_tree_dense_mask": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p]),
    "pst_last_error": (c_char_p, []),
    "pst_build_sources_sha256": (c_char_p, []),
}

_lib = None


def header_functions():
    """Names of the functions include/pst.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(pst_\w+)\s*\(", text, re.M)))


def verify_build(lib, want: str) -> None:
    """Raise unless `lib` was built from the sources whose digest is `want`."""
    got = lib.pst_build_sources_sha256().decode()
    if got != want:
        raise RuntimeError(f"libpst was built from other sources (digest {got[:16]}, sources "
                           f"{want[:16]}); rebuild: python -m prefix_shared_tree_packed_amd.build")


def load(path: str = LIB_PATH):
    """Load libpst.so (built in-tree).  Raises if it is missing (there is no
    fallback implementation) or, for the in-tree library, if it was built
    from sources other than the ones in the tree."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m prefix_shared_tree_packed_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        # a build without the device entry points (the host-only sanitizer
        # build) leaves them undeclared: calling one raises AttributeError
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    if path == os.path.join(PKG, "libpst.so"):
        from .build import sources_sha256
        verify_build(lib, sources_sha256())
    _lib = lib
    return lib


class PstError(RuntimeError):
    def __init__(self, code: int, message: str):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        super().__init__(f"{self.name}: {message}")


def check(code: int):
    if code != PST_OK:
        raise PstError(code, load().pst_last_error().decode())
