"""CPU oracle for tree-verification attention (and the D-cut and E2E-TV
steps next to it: D-cut selection, E2E-TV statistics, Graft retrieval and
its online table update, stochastic tree verification) -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports it, and it imports
nothing from the product path.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    mask_bits,
    mask_anchor,
    tree_attn,
    accept,
    dcut_select,
    e2e_tv_stats,
    graft_retrieve,
    graft_update,
    accept_sampled,
)
