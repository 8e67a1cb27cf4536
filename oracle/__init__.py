"""CPU oracle for prefix-shared tree training — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation (numpy, float64) of what the
tree-training hot path computes, written from the AReaL tree-training page
("树训练": sections 树构建过程, TrieNode, 对数概率计算, 注意力机制, 指标和监控).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP library and imports nothing
from it; the library never calls back into it.

Modules:
  tree        sequence intake, first-fit-decreasing trie packing, chain
              compression, preorder flattening, padding, tile classes
  attention   dense ancestor mask, masked-softmax attention forward/backward
  gather      per-sequence next-token log-probabilities and entropies, and
              their gradient with respect to the packed logits
  accounting  tree_token_ratio, visible pairs, FLOP counts
  rope        rotary position embedding with pos = depth
  packing     FFD and Karmarkar-Karp allocation of items (sequences, trees)
              to micro-batches or ranks, and the packing-quality metrics
              (from the article on AReaL's FFD/KK packing)
"""

from .tree import (  # noqa: F401
    OracleError, InvalidInput, CapacityError, BlockError,
    Node, Tree, Forest, build_forest, BLOCK,
)
from .attention import (  # noqa: F401
    ancestors, dense_mask, attn_fwd, attn_bwd, attn_bwd_magnitudes, attn_fwd_rows, attn_bwd_rows,
)
from .gather import (  # noqa: F401
    gather_logprobs_entropy, gather_logprobs_entropy_bwd, row_lse_entropy,
)
from .accounting import forest_stats, attn_flops  # noqa: F401
from .rope import rope  # noqa: F401
from . import packing  # noqa: F401
