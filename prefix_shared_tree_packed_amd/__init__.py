"""prefix_shared_tree_packed_amd: the MI355X (gfx950) hot path of
prefix-shared tree training behind the C ABI of include/pst.h.

Importing the package does not load the library; the first call does, and
fails loudly if libpst.so has not been built (there is no CPU fallback).
"""

from ._lib import PstError, load, header_functions  # noqa: F401
from .api import (  # noqa: F401
    Forest,
    TreeMeta,
    build_tree,
    tree_meta_create,
    forest_meta_create,
    tree_attn_fwd,
    tree_attn_bwd,
    tree_attn_bwd_workspace_bytes,
    tree_attn_bwd_noalloc,
    gather_tree_logprobs_entropy,
    gather_tree_logprobs_entropy_bwd,
    tree_rope,
    PACKING_ALGORITHMS,
    pack_allocate,
    packing_metrics,
    assign_trees,
    MASK_FORMATS,
    tree_dense_mask,
)
