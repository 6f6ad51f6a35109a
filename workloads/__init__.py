"""Seeded synthetic workloads for tree-verification attention.

This package only draws inputs (trees, token ids, Q/K/V, page tables, and for
sampled verification the two models' logits and the uniforms).  It
holds none of the arithmetic of the verification path (no mask building, no
attention, no acceptance), so both the HIP path and the CPU oracle can take
their inputs from it. (The config-3 recipe cuts its chains with a float64
prefix-product ranking: that shapes the input trees only; the device D-cut
selection is checked against the oracle, never against this.)
"""
from .configs import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    GRAFT_TREE_PARENT,
    QWEN3_VOCAB,
    build_workload,
    make,
    random_tree,
    trunk_branch_tree,
)
from .sampled import SampledInputs, sampled_inputs  # noqa: F401
