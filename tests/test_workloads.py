"""Checks of the seeded generators against the shapes the pages fix (CPU only)."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def depths(par):
    d = [0] * len(par)
    for i in range(1, len(par)):
        d[i] = d[par[i]] + 1
    return d


def test_graft_tree_matches_depth5_budget_split():
    with open(os.path.join(GOLDEN, "graft_budget_split.json")) as f:
        g = json.load(f)
    par = W.GRAFT_TREE_PARENT
    n_draft, n_retr = g["split_draft_retrieved"]["prune_at_depth_5"]
    assert len(par) == g["budget"] == n_draft + n_retr
    d = depths(par)
    # draft part: nodes 0..39, depths 0..5 with level sizes 1, 3, 9, 9, 9, 9
    assert [d[:n_draft].count(k) for k in range(6)] == [1, 3, 9, 9, 9, 9]
    # retrieved part hangs entirely below one depth-5 draft node (the prune checkpoint)
    graft = par[n_draft]
    assert d[graft] == 5 == g["checkpoint_depths"][-1]
    for i in range(n_draft, len(par)):
        j = i
        while j >= n_draft:
            j = par[j]
        assert j == graft
    assert max(d) == 10 and sum(x + 1 for x in d) == 343


def test_dcut_generator_budget_and_contiguous_prefixes():
    with open(os.path.join(GOLDEN, "dcut_budget.json")) as f:
        g = json.load(f)
    w = W.make(3, batch=16, prefix_range=(10, 40))
    block = g["draft_length"] + 1
    assert w.meta["rho"] in g["rho_grid"]
    assert w.total_nodes == w.meta["budget"] == int(w.meta["rho"] * 16 * block)
    for b in range(w.batch):
        par = w.parent[w.cu_nodes[b]:w.cu_nodes[b + 1]]
        assert par.tolist() == [-1] + list(range(len(par) - 1))      # a chain prefix
        assert 1 <= len(par) <= block


def test_specopd_tree_shape():
    w = W.make(5, trunk=256, n_anchors=6, width=16, anchor_lo=64)
    anchors = w.meta["anchors"]
    assert (np.diff(anchors) > 0).all() and anchors.min() >= 64 and anchors.max() < 256
    assert w.total_nodes == 256 + 6 * 16 and w.prefix_len.tolist() == [0]
    par = w.parent
    assert par[:256].tolist() == [-1] + list(range(255))
    for j, a in enumerate(anchors):
        s = 256 + 16 * j
        assert par[s] == a and par[s + 1:s + 16].tolist() == list(range(s, s + 15))


def test_generators_are_seeded_and_deterministic():
    a = W.make(2, prefix=100)
    b = W.make(2, prefix=100)
    assert (a.draft_tok == b.draft_tok).all() and (a.target_tok == b.target_tok).all()
    assert (a.k_cache == b.k_cache).all() and (a.q == b.q).all()
    c = W.make(2, seed=99, prefix=100)
    assert not (a.q == c.q).all()


def test_config1_tree_shape():
    w = W.make(1)
    par = w.parent.tolist()
    d = depths(par)
    assert len(par) == 15 and max(d) == 4 and par[:4] == [-1, 0, 0, 0]
    assert sum(1 for p in par if p == 0) == 3


def test_permuted_pool_is_a_permutation():
    w = W.make(4, batch=2, prefix=100)
    used = w.block_table[w.block_table >= 0]
    assert len(set(used.tolist())) == used.size == w.num_pages
