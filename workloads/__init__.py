"""Seeded synthetic inputs for the prefix-shared tree path.

This package only draws random token sequences and tensors. It contains none
of the method's arithmetic (no trie, no masks, no attention, no softmax), so
both the CPU oracle and the HIP path may take their inputs from it.
"""

from .configs import (  # noqa: F401
    Workload,
    WORKLOADS,
    get_workload,
    worked_example,
    worked_example_edge,
    make_tensor,
    tree_tensor_seed,
    bimodal_lengths,
)
