"""MI355X (gfx950) tree-verification attention: mask build, verify attention, greedy accept
and stochastic (recursive rejection sampling) acceptance, the D-cut verification budget that packs chain drafts ahead of them, and SpecOPD's
E2E-TV statistics after them, and Graft's retrieval table (template expansion and
online update).

The calls are thin wrappers over the C ABI of ``lib/libtreeverify.so``
(``include/treeverify.h``); build it with
``python -m tree_verification_attention_mask_amd.build``.
"""
from .binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    TVError,
    dcut_select,
    e2e_tv_stats,
    graft_retrieve,
    graft_update,
    graft_update_workspace_size,
    load_library,
    mask_struct,
    tree_accept,
    tree_accept_sampled,
    tree_accept_sampled_workspace_size,
    tree_mask_build,
    tree_verify_attn,
    tree_verify_attn_noalloc,
    verify_attn_plan,
    verify_attn_workspace_size,
)
