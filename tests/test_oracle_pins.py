"""Pins of the CPU oracle to facts fixed outside it (no GPU needed).

Each test checks the oracle against something the pages or the mathematics
fix independently of its C code: a worked illustration from a page, a closed
form, a special case that a library routine computes (torch's
scaled_dot_product_attention in float64), an invariant the pages state, or a
brute force written differently (boolean matrix closure, greedy descent).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def closure(parent):
    """Reflexive-transitive closure of child->parent by boolean matrix powers."""
    n = len(parent)
    A = np.zeros((n, n), bool)
    for i in range(1, n):
        A[i, parent[i]] = True
    R = np.eye(n, dtype=bool)
    while True:
        R2 = R | ((R.astype(np.int64) @ A.astype(np.int64)) > 0)
        if (R2 == R).all():
            return R
        R = R2


def bits_to_dense(bits, n):
    out = np.zeros((n, n), bool)
    for i in range(n):
        for j in range(n):
            out[i, j] = (int(bits[i, j // 64]) >> (j % 64)) & 1
    return out


# ------------------------------------------------------------------ masks --

def test_mask_chain_is_lower_triangular(oracle_lib):
    n = 100
    par = [-1] + list(range(n - 1))
    bits, depth, err = oracle.mask_bits(par, [0, n], 2)
    assert err.tolist() == [0]
    assert (bits_to_dense(bits, n) == np.tril(np.ones((n, n), bool))).all()
    assert depth.tolist() == list(range(n))


def test_mask_star_is_diagonal_plus_root(oracle_lib):
    n = 40
    par = [-1] + [0] * (n - 1)
    bits, depth, err = oracle.mask_bits(par, [0, n], 1)
    expect = np.eye(n, dtype=bool)
    expect[:, 0] = True
    assert (bits_to_dense(bits, n) == expect).all()
    assert depth.tolist() == [0] + [1] * (n - 1)


@pytest.mark.parametrize("seed", range(6))
def test_mask_matches_matrix_closure(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    trees = [W.random_tree(rng, int(n)) for n in rng.integers(1, 200, size=4)]
    cu = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    bits, depth, err = oracle.mask_bits(np.concatenate(trees), cu, 4)
    assert (err == 0).all()
    for b, t in enumerate(trees):
        R = closure(t)
        got = bits_to_dense(bits[cu[b]:cu[b + 1]], len(t))
        assert (got == R).all()
        assert (depth[cu[b]:cu[b + 1]] == R.sum(1) - 1).all()


@pytest.mark.parametrize("bad", [
    [0, 0, 1],          # root does not have parent -1
    [-1, 0, 2],         # parent equal to self
    [-1, 0, 3, 1],      # parent after the node (would allow a cycle)
    [-1, 0, -1],        # a second root
    [-1, -2, 0],        # out of range
])
def test_mask_rejects_malformed_trees(oracle_lib, bad):
    good = [-1, 0, 0, 1]
    par = np.array(good + bad, np.int32)
    cu = [0, len(good), len(good) + len(bad)]
    bits, depth, err = oracle.mask_bits(par, cu, 1)
    assert err.tolist() == [0, 1]
    assert (bits[len(good):] == 0).all() and (depth[len(good):] == -1).all()
    ap, bd, dep, err2 = oracle.mask_anchor(par, cu)
    assert err2.tolist() == [0, 1]


def test_mask_rejects_tree_wider_than_words(oracle_lib):
    n = 65
    par = [-1] + list(range(n - 1))
    _, _, err = oracle.mask_bits(par, [0, n], 1)
    assert err.tolist() == [1]


@pytest.mark.parametrize("seed", range(5))
def test_anchor_form_equals_closure(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    trees = []
    for _ in range(3):
        trunk = int(rng.integers(1, 120))
        nb = int(rng.integers(0, 8))
        anchors = np.sort(rng.integers(0, trunk, size=nb))
        if nb:
            anchors[-1] = trunk - 1          # a branch at the last trunk node
        par = W.trunk_branch_tree(trunk, anchors.tolist(), int(rng.integers(1, 20)))
        trees.append(par)
    cu = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    ap, bd, depth, err = oracle.mask_anchor(np.concatenate(trees), cu)
    assert (err == 0).all()
    for b, t in enumerate(trees):
        n = len(t)
        R = closure(t)
        a, d = ap[cu[b]:cu[b + 1]], bd[cu[b]:cu[b + 1]]
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        vis = (j <= a[:, None]) | ((j > i - d[:, None]) & (j <= i))
        assert (vis == R).all()
        assert (depth[cu[b]:cu[b + 1]] == R.sum(1) - 1).all()


def test_anchor_form_rejects_branch_of_branch(oracle_lib):
    par = W.trunk_branch_tree(10, [3, 7], 4)
    par.append(len(par) - 3)                # hangs off the middle of a branch
    _, _, _, err = oracle.mask_anchor(par, [0, len(par)])
    assert err.tolist() == [2]


# -------------------------------------------------------------- attention --

def gathered_kv(w, b):
    """Contiguous [Hkv, P+n, D] float64 K and V of request b, read through its page table."""
    L = int(w.prefix_len[b]) + int(w.nodes_per_request[b])
    pos = np.arange(L)
    pages = torch.from_numpy(w.block_table[b, pos // w.page_size].astype(np.int64))
    slots = torch.from_numpy(pos % w.page_size)
    k = w.k_cache.double()[pages, :, slots, :].permute(1, 0, 2)
    v = w.v_cache.double()[pages, :, :, slots].permute(1, 0, 2)
    return k, v


def sdpa_reference(w, b, vis_tree):
    """torch float64 SDPA for request b with boolean tree visibility [n, n];
    prefix keys visible to every node; KV heads repeated per GQA group."""
    P, n = int(w.prefix_len[b]), int(w.nodes_per_request[b])
    k, v = gathered_kv(w, b)
    G = w.num_q_heads // w.num_kv_heads
    k = k.repeat_interleave(G, 0)
    v = v.repeat_interleave(G, 0)
    q = w.q.double()[w.cu_nodes[b]:w.cu_nodes[b + 1]].permute(1, 0, 2)   # [Hq, n, D]
    mask = torch.cat([torch.ones(n, P, dtype=torch.bool), torch.from_numpy(vis_tree)], 1)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale)
    s = (q @ k.transpose(1, 2)) * w.scale
    s = s.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(s, -1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


def small(parent_lists, prefix, hq=8, hkv=2, d=32, seed=0, **kw):
    return W.build_workload("pin", parent_lists, prefix, hq, hkv, d, "f32", seed, **kw)


def test_chain_tree_equals_causal_attention(oracle_lib):
    n, P = 23, 37
    w = small([[-1] + list(range(n - 1))], [P], seed=1, permute_pages=True)
    out, lse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.cu_nodes, w.parent, 8, 2, w.scale)
    ref, rlse = sdpa_reference(w, 0, np.tril(np.ones((n, n), bool)))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_tree_attention_equals_sdpa_with_closure_mask(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    trees = [W.random_tree(rng, int(n), max_children=4) for n in (1, 17, 60)]
    prefix = [int(p) for p in rng.integers(0, 90, size=3)]
    w = small(trees, prefix, hq=6, hkv=3, d=16, seed=seed, permute_pages=True, spare_pages=3)
    for form in ("dense", "path"):
        out, lse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                    w.cu_nodes, w.parent, 6, 3, w.scale, formulation=form)
        for b, t in enumerate(trees):
            ref, rlse = sdpa_reference(w, b, closure(t))
            sl = slice(w.cu_nodes[b], w.cu_nodes[b + 1])
            np.testing.assert_allclose(out[sl], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[sl], rlse, rtol=0, atol=1e-12)


def test_single_node_no_prefix_returns_its_own_value(oracle_lib):
    w = small([[-1]], [0], seed=3)
    out, lse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.cu_nodes, w.parent, 8, 2, w.scale)
    for h in range(8):
        g = h // 4
        np.testing.assert_array_equal(out[0, h], w.v_cache[0, g, :, 0].double().numpy())
        s = float((w.q[0, h].double() * w.k_cache[0, g, 0].double()).sum()) * w.scale
        assert abs(lse[0, h] - s) < 1e-12


def test_equal_keys_give_mean_of_visible_values(oracle_lib):
    rng = np.random.default_rng(7)
    tree = W.random_tree(rng, 30)
    P = 50
    w = small([tree], [P], seed=7)
    w.k_cache[:] = w.k_cache[0, :, 0:1, :]     # every key of a kv head identical
    out, lse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.cu_nodes, w.parent, 8, 2, w.scale)
    k, v = gathered_kv(w, 0)
    R = closure(tree)
    for i in range(len(tree)):
        keys = list(range(P)) + [P + j for j in range(len(tree)) if R[i, j]]
        for h in range(8):
            g = h // 4
            np.testing.assert_allclose(out[i, h], v[g, keys].mean(0).numpy(), atol=1e-12)
            s = float((w.q[i, h].double() * k[g, 0]).sum()) * w.scale
            assert abs(lse[i, h] - (s + math.log(len(keys)))) < 1e-12


def test_gqa_group_shares_one_kv_head(oracle_lib):
    rng = np.random.default_rng(11)
    w = small([W.random_tree(rng, 20)], [40], hq=8, hkv=2, seed=11)
    w.q[:, 1:4] = w.q[:, 0:1]                  # heads 0..3 = group 0
    w.q[:, 5:8] = w.q[:, 4:5]                  # heads 4..7 = group 1
    out, lse = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                                w.cu_nodes, w.parent, 8, 2, w.scale)
    for h in (1, 2, 3):
        np.testing.assert_array_equal(out[:, h], out[:, 0])
    for h in (5, 6, 7):
        np.testing.assert_array_equal(out[:, h], out[:, 4])
    assert np.abs(out[:, 0] - out[:, 4]).max() > 1e-3   # the two groups differ


def test_non_ancestor_kv_does_not_matter(oracle_lib):
    tree = [-1, 0, 0, 1, 1, 2, 2, 3]
    P = 20
    w = small([tree], [P], seed=5)
    base, _ = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                               w.cu_nodes, w.parent, 8, 2, w.scale)
    R = closure(tree)
    j = 2                                       # perturb node 2's K and V
    pos = P + j
    page, slot = w.block_table[0, pos // 16], pos % 16
    w.k_cache[page, :, slot] += 3.0
    w.v_cache[page, :, :, slot] -= 2.0
    out, _ = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_len,
                              w.cu_nodes, w.parent, 8, 2, w.scale)
    for i in range(len(tree)):
        if R[i, j]:
            assert np.abs(out[i] - base[i]).max() > 1e-6
        else:
            np.testing.assert_array_equal(out[i], base[i])


def test_page_permutation_and_row_subset_do_not_change_results(oracle_lib):
    rng = np.random.default_rng(9)
    tree = W.random_tree(rng, 33)
    a = small([tree], [75], seed=9)
    b = small([tree], [75], seed=9, permute_pages=True)
    # same values, different placement: move b's pages so logical content matches a
    for blk in range(a.block_table.shape[1]):
        b.k_cache[b.block_table[0, blk]] = a.k_cache[a.block_table[0, blk]]
        b.v_cache[b.block_table[0, blk]] = a.v_cache[a.block_table[0, blk]]
    b.q.copy_(a.q)
    oa, la = oracle.tree_attn(a.q, a.k_cache, a.v_cache, a.block_table, a.prefix_len,
                              a.cu_nodes, a.parent, 8, 2, a.scale)
    ob, lb = oracle.tree_attn(b.q, b.k_cache, b.v_cache, b.block_table, b.prefix_len,
                              b.cu_nodes, b.parent, 8, 2, b.scale)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
    rows = np.array([[0, 0], [32, 7], [5, 3]], np.int32)
    orow, lrow = oracle.tree_attn(a.q, a.k_cache, a.v_cache, a.block_table, a.prefix_len,
                                  a.cu_nodes, a.parent, 8, 2, a.scale, rows=rows)
    for r, (i, h) in enumerate(rows):
        np.testing.assert_array_equal(orow[r], oa[i, h])
        assert lrow[r] == la[i, h]


# ------------------------------------------------------------- acceptance --

def chain_case(correct, seed=0):
    """Root + len(correct) drafted nodes; drafted token k is right iff correct[k-1]."""
    rng = np.random.default_rng(seed)
    n = len(correct) + 1
    par = [-1] + list(range(n - 1))
    draft = rng.integers(1000, size=n).astype(np.int32)
    target = rng.integers(1000, size=n).astype(np.int32)
    for k in range(1, n):
        target[k - 1] = draft[k] if correct[k - 1] else (draft[k] + 1) % 1000
    return par, draft, target


def test_specopd_illustration_golden(oracle_lib):
    with open(os.path.join(GOLDEN, "specopd_al_illustration.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        par, dr, tg = chain_case(case["token_correct"])
        al, path, bonus = oracle.accept(par, dr, tg, [0, len(par)], len(par) - 1)
        assert al[0] == case["acceptance_length"], case["name"]


@pytest.mark.parametrize("seed", range(10))
def test_chain_acceptance_is_prefix_survival(oracle_lib, seed):
    # BlockPilot §八: accepted length = sum_k prod_{j<=k} alpha_j; with the 0/1
    # outcome of each position this is the index of the first mismatch.
    rng = np.random.default_rng(seed)
    correct = (rng.random(int(rng.integers(1, 25))) < 0.8)
    par, dr, tg = chain_case(correct, seed)
    al, path, bonus = oracle.accept(par, dr, tg, [0, len(par)], len(par) - 1)
    survival = sum(np.prod(correct[:k + 1].astype(int)) for k in range(len(correct)))
    first_miss = int(np.argmin(np.append(correct, False)))
    assert al[0] == survival == first_miss
    assert path[0, :al[0] + 1].tolist() == list(range(al[0] + 1))
    assert (path[0, al[0] + 1:] == -1).all()
    assert bonus[0] == tg[al[0]]


def greedy_descent(par, dr, tg):
    ch = [[] for _ in par]
    for i in range(1, len(par)):
        ch[par[i]].append(i)
    cur, path = 0, [0]
    while True:
        nxt = [c for c in ch[cur] if dr[c] == tg[cur]]
        if not nxt:
            return path, tg[cur]
        cur = nxt[0]
        path.append(cur)


@pytest.mark.parametrize("seed", range(8))
def test_distinct_siblings_acceptance_equals_greedy_descent(oracle_lib, seed):
    w = W.build_workload("acc", [W.random_tree(np.random.default_rng(seed), int(n))
                                 for n in (1, 9, 60, 200)],
                         [0, 0, 0, 0], 2, 1, 8, "f32", seed, vocab=50, match_p=0.8)
    md = w.max_depth
    al, path, bonus = oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes, md)
    for b in range(w.batch):
        sl = slice(w.cu_nodes[b], w.cu_nodes[b + 1])
        gp, gb = greedy_descent(w.parent[sl], w.draft_tok[sl], w.target_tok[sl])
        assert al[b] == len(gp) - 1
        assert path[b, :len(gp)].tolist() == gp
        assert bonus[b] == gb


@pytest.mark.parametrize("seed", range(6))
def test_appending_nodes_never_shortens_acceptance(oracle_lib, seed):
    # Graft §三: a superset tree never has a shorter longest accepted prefix.
    rng = np.random.default_rng(seed)
    par = W.random_tree(rng, 30)
    dr = list(rng.integers(6, size=30))
    tg = list(rng.integers(6, size=30))
    prev = oracle.accept(par, dr, tg, [0, len(par)], 200)[0][0]
    for _ in range(40):
        par.append(int(rng.integers(len(par))))
        dr.append(int(rng.integers(6)))
        tg.append(int(rng.integers(6)))
        cur = oracle.accept(par, dr, tg, [0, len(par)], 200)[0][0]
        assert cur >= prev
        prev = cur


def test_empty_requests_accept_nothing_and_leave_the_others_alone(oracle_lib):
    # A request with no nodes has no root, so nothing is accepted: length 0,
    # an all -1 path and no bonus token (-1). Every other request of the batch
    # gets exactly what it gets alone, whether the empty ones come first, in
    # the middle or last (the read of the next request's nodes is the mistake
    # this guards against).
    rng = np.random.default_rng(11)
    trees = [W.random_tree(rng, n) for n in (7, 1, 30)]
    toks = [(list(rng.integers(4, size=len(t))), list(rng.integers(4, size=len(t))))
            for t in trees]
    alone = [oracle.accept(t, d, g, [0, len(t)], 12) for t, (d, g) in zip(trees, toks)]
    for layout in ([None, 0, 1, 2], [0, None, None, 1, 2], [0, 1, 2, None]):
        par, dr, tg, cu = [], [], [], [0]
        for k in layout:
            if k is not None:
                par += trees[k]
                dr += toks[k][0]
                tg += toks[k][1]
            cu.append(len(par))
        al, path, bonus = oracle.accept(par, dr, tg, cu, 12)
        for b, k in enumerate(layout):
            if k is None:
                assert al[b] == 0 and bonus[b] == -1 and (path[b] == -1).all(), layout
            else:
                assert al[b] == alone[k][0][0] and bonus[b] == alone[k][2][0], layout
                np.testing.assert_array_equal(path[b], alone[k][1][0])


def test_repeated_sibling_tokens_pick_deepest_then_smallest_index(oracle_lib):
    # root -> {1, 2} both carry token 7 and both match; 2 has an accepted child.
    par = [-1, 0, 0, 2, 1]
    dr = [0, 7, 7, 9, 9]
    tg = [7, 9, 9, 0, 0]
    al, path, bonus = oracle.accept(par, dr, tg, [0, 5], 4)
    assert al[0] == 2 and path[0, :3].tolist() == [0, 2, 3]   # 3 (via 2) ties 4 (via 1): smaller index
    assert bonus[0] == tg[3]
    par2 = [-1, 0, 0, 2]
    dr2 = [0, 7, 7, 9]
    tg2 = [7, 0, 9, 0]
    al2, path2, _ = oracle.accept(par2, dr2, tg2, [0, 4], 3)
    assert al2[0] == 2 and path2[0, :3].tolist() == [0, 2, 3]


# ---------------------------------------------------------------------------
# D-cut selection (D-cut technical summary §2: prefix-product scores, one
# global ranking over the batch, kept positions packed as per-request prefixes)

def _dcut(conf, budget, tokens=None):
    conf = np.asarray(conf, np.float32)
    b, d = conf.shape
    if tokens is None:
        tokens = np.arange(b * (d + 1), dtype=np.int32).reshape(b, d + 1)
    return oracle.dcut_select(conf, tokens, budget)


def test_dcut_extreme_budgets(oracle_lib):
    rng = np.random.default_rng(1)
    conf = rng.uniform(0.1, 1.0, size=(5, 7))
    n, cu, par, tok = _dcut(conf, 5)                       # only the current tokens
    assert n.tolist() == [1] * 5 and cu.tolist() == list(range(6)) and par.tolist() == [-1] * 5
    n, cu, par, tok = _dcut(conf, 5 * 8)                   # every drafted token
    assert n.tolist() == [8] * 5
    for bad in (4, 41):
        with pytest.raises(ValueError):
            _dcut(conf, bad)


@pytest.mark.parametrize("budget", [9, 12, 13, 20, 31])
def test_dcut_equal_confidences_fill_depth_by_depth(oracle_lib, budget):
    # equal confidences: the score depends on depth only, so the extra slots
    # go one depth at a time, requests in order (closed form)
    B, D = 6, 5
    n = _dcut(np.full((B, D), 0.75), budget)[0]
    q, r = divmod(budget - B, B)
    assert n.tolist() == [1 + q + (b < r) for b in range(B)]


@pytest.mark.parametrize("seed", range(8))
def test_dcut_keeps_the_best_prefix_set_by_brute_force(oracle_lib, seed):
    # among all per-request prefix lengths with the same total, the kept set
    # has the largest total score (scores distinct here, so it is unique)
    import itertools
    rng = np.random.default_rng(seed)
    B, D = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.uniform(0.05, 1.0, size=(B, D)).astype(np.float32)
    score = np.ones((B, D + 1), np.float64)
    score[:, 1:] = np.cumprod(conf, axis=1, dtype=np.float32)
    for budget in range(B, B * (D + 1) + 1):
        best, arg = -1.0, None
        for ns in itertools.product(range(1, D + 2), repeat=B):
            if sum(ns) != budget:
                continue
            tot = sum(score[b, :ns[b]].sum() for b in range(B))
            if tot > best + 1e-12:
                best, arg = tot, ns
        assert _dcut(conf, budget)[0].tolist() == list(arg)


@pytest.mark.parametrize("seed", range(4))
def test_dcut_one_more_slot_adds_one_position(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    conf = rng.beta(4.0, 2.0, size=(9, 15))
    prev = _dcut(conf, 9)[0]
    for budget in range(10, 9 * 16 + 1):
        cur = _dcut(conf, budget)[0]
        diff = cur - prev
        assert diff.min() == 0 and diff.sum() == 1
        prev = cur


def test_dcut_agrees_with_the_config3_recipe(oracle_lib):
    # the config-3 generator ranks the same scores in float64 with its own sort;
    # away from near-ties both give the same per-request lengths
    w = W.make(3)
    conf = np.asarray(w.meta["confidence"], np.float64)
    n = _dcut(conf.astype(np.float32), w.meta["budget"])[0]
    assert n.tolist() == [int(x) for x in w.nodes_per_request]


def test_dcut_confidences_are_probabilities(oracle_lib):
    # NaN / negative -> 0 and > 1 -> 1: a 0 ends a block's scores, a 1 keeps them
    conf = np.array([[np.nan, 0.9, 0.9], [1.5, 0.6, 0.5], [-2.0, 1.0, 1.0], [0.8, 0.1, 0.1]],
                    np.float32)
    n = _dcut(conf, 4 + 2)[0]
    # request 1 scores 1.0, 0.6, 0.3 (not 1.5, 0.9, ...), request 3 0.8, 0.08, ...
    assert n.tolist() == [1, 2, 1, 2]


def test_dcut_packs_prefixes_in_request_order(oracle_lib):
    rng = np.random.default_rng(7)
    conf = rng.uniform(0.2, 1.0, size=(4, 6))
    tokens = rng.integers(0, 10 ** 6, size=(4, 7)).astype(np.int32)
    n, cu, par, tok = _dcut(conf, 15, tokens)
    assert cu.tolist() == [0] + np.cumsum(n).tolist()
    for b in range(4):
        seg = slice(cu[b], cu[b + 1])
        assert tok[seg].tolist() == tokens[b, :n[b]].tolist()
        assert par[seg].tolist() == list(range(-1, n[b] - 1))


# ---------------------------------------------------------------------------
# SpecOPD E2E-TV statistics (SpecOPD §02 stage 4, §03.2): alpha = overlap of
# the target and draft next-token distributions = 1 - TV; prefix products
# along a branch; expected run of accepted tokens = their sum

def test_e2e_alpha_is_one_minus_total_variation(oracle_lib):
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    t = rng.normal(0, 2, size=(6, 300))
    d = t + rng.normal(0, 1, size=(6, 300))
    alpha = oracle.e2e_tv_stats(t, d, [0, 6])[0]
    tv_dist = 0.5 * np.abs(softmax(t, axis=1) - softmax(d, axis=1)).sum(axis=1)
    np.testing.assert_allclose(alpha, 1.0 - tv_dist, rtol=0, atol=1e-12)


def test_e2e_alpha_special_cases(oracle_lib):
    rng = np.random.default_rng(12)
    t = rng.normal(0, 3, size=(3, 64))
    # identical distributions (also after a constant shift of the logits): 1
    a = oracle.e2e_tv_stats(t, t + 5.0, [0, 3])[0]
    np.testing.assert_allclose(a, 1.0, atol=1e-12)
    # disjoint supports: 0
    big = np.full((1, 8), -1e4)
    t1, d1 = big.copy(), big.copy()
    t1[0, 0] = 0.0
    d1[0, 1] = 0.0
    assert oracle.e2e_tv_stats(t1, d1, [0, 1])[0][0] < 1e-12
    # two tokens: p = (a, 1-a), q = (b, 1-b) -> 1 - |a - b|
    for pa, qb in [(0.3, 0.8), (0.5, 0.5), (0.99, 0.01)]:
        t2 = np.log([[pa, 1 - pa]])
        d2 = np.log([[qb, 1 - qb]])
        got = oracle.e2e_tv_stats(t2, d2, [0, 1])[0][0]
        assert abs(got - (1 - abs(pa - qb))) < 1e-12


def test_e2e_temperature_scales_the_logits(oracle_lib):
    rng = np.random.default_rng(13)
    t = rng.normal(0, 2, size=(4, 100))
    d = rng.normal(0, 2, size=(4, 100))
    a_t = oracle.e2e_tv_stats(t, d, [0, 4], temperature=2.5)[0]
    a_1 = oracle.e2e_tv_stats(t / 2.5, d / 2.5, [0, 4], temperature=1.0)[0]
    np.testing.assert_allclose(a_t, a_1, atol=1e-12)
    hot = oracle.e2e_tv_stats(t, d, [0, 4], temperature=1e6)[0]   # both near uniform
    assert (hot > 1 - 1e-4).all()


@pytest.mark.parametrize("w", [1, 4, 16])
def test_e2e_chain_of_equal_alphas_is_a_geometric_series(oracle_lib, w):
    t2 = np.log([[0.3, 0.7]] * w)
    d2 = np.log([[0.6, 0.4]] * w)                 # alpha = 1 - 0.3 = 0.7 at every node
    alpha, prefix, expected = oracle.e2e_tv_stats(t2, d2, [0, w])
    a = 0.7
    np.testing.assert_allclose(prefix, [a ** k for k in range(1, w + 1)], atol=1e-12)
    assert abs(expected[0] - a * (1 - a ** w) / (1 - a)) < 1e-12
    # branches are independent: splitting the same nodes into two branches
    if w > 1:
        _, p2, e2 = oracle.e2e_tv_stats(t2, d2, [0, 1, w])
        assert abs(e2[0] - a) < 1e-12 and abs(p2[1] - a) < 1e-12


# ---------------------------------------------------------------------------
# Graft retrieval and online update (Graft §二 second and third gear, §五):
# a device table of each token's top-k successors, a template expanded from
# the current token, rows replaced by the target's top-k after verification

def _succ_table(v, k, step=1):
    """Row t lists t+step, t+2*step, ... (mod v): successors with a closed form."""
    return np.array([[(t + step * (r + 1)) % v for r in range(k)] for t in range(v)], np.int32)


def test_graft_retrieve_follows_ranks_along_the_template(oracle_lib):
    v, k = 97, 4
    adj = _succ_table(v, k)
    # chain of depth 5 taking ranks 0, 2, 1, 3, 0, a second child of the root,
    # and a node hanging under the chain's second node (not the node before it)
    par = [-1, 0, 1, 2, 3, -1, 1]
    rank = [0, 2, 1, 3, 0, 2, 1]
    out = oracle.graft_retrieve(adj, [5, 90], par, rank)
    for b, root in enumerate([5, 90]):
        t, exp = root, []
        for r in rank[:5]:
            t = (t + r + 1) % v
            exp.append(t)
        exp.append((root + 3) % v)
        exp.append((exp[1] + 2) % v)     # under node 1 (token root+4), not node 5 (root+3)
        assert out[b].tolist() == exp


def test_graft_retrieve_missing_entries_empty_the_subtree(oracle_lib):
    v, k = 20, 3
    adj = _succ_table(v, k)
    adj[6, 1] = -1                      # token 6 lacks its second successor
    adj[7, 0] = 99                      # out of the vocabulary
    par, rank = [-1, 0, 1, -1, 3], [0, 0, 0, 1, 0]
    out = oracle.graft_retrieve(adj, [5, 6, -3], par, rank)
    # from 5: 6, then 7, then adj[7][0] = 99 (out of range) -> -1; 5's 2nd is 7 -> -1 below
    assert out[0].tolist() == [6, 7, -1, 7, -1]
    # from 6: 7, -1, -1; 6's 2nd successor is missing, so its child is too
    assert out[1].tolist() == [7, -1, -1, -1, -1]
    assert out[2].tolist() == [-1] * 5              # no current token


def test_graft_update_takes_the_targets_top_k(oracle_lib):
    rng = np.random.default_rng(21)
    v, k = 1000, 8
    adj = _succ_table(v, k)
    centre = [100, 500, 999]
    u = np.arange(v)
    # logits falling with the distance from a centre (plus a tiny tie-breaking
    # slope): the top-k are the k tokens nearest the centre, nearest first
    logits = np.stack([-np.abs(u - c) - 1e-3 * u for c in centre]).astype(np.float32)
    new = oracle.graft_update(adj, logits, [3, 4, 5])
    for row, c in zip((3, 4, 5), centre):
        near = sorted(u, key=lambda x: (abs(x - c), x))[:k]
        assert new[row].tolist() == near
    untouched = np.setdiff1d(u, [3, 4, 5])
    np.testing.assert_array_equal(new[untouched], adj[untouched])
    flat = oracle.graft_update(adj, np.zeros((1, v), np.float32), [7])
    assert flat[7].tolist() == list(range(k))       # all equal: smallest ids


def test_graft_update_later_node_wins_and_nan_ranks_last(oracle_lib):
    v, k = 50, 3
    adj = _succ_table(v, k)
    lg = np.full((3, v), -5.0, np.float32)
    lg[0, 10] = 1.0
    lg[1, 20] = 1.0
    lg[2, [30, 31]] = np.nan
    lg[2, 40] = 2.0
    new = oracle.graft_update(adj, lg, [9, 9, 11])
    assert new[9].tolist() == [20, 0, 1]            # node 1 (later) wins row 9
    assert new[11].tolist() == [40, 0, 1]           # NaNs never outrank finite logits
    assert oracle.graft_update(adj, lg, [-1, 50, 1000]).tolist() == adj.tolist()


def test_graft_update_then_retrieve_follows_the_new_rows(oracle_lib):
    v, k = 64, 2
    adj = np.full((v, k), -1, np.int32)
    lg = np.full((3, v), -1.0, np.float32)
    lg[0, 11] = 1.0        # after token 10 the target expects 11, then 12 ...
    lg[1, 12] = 1.0
    lg[2, 13] = 1.0
    adj = oracle.graft_update(adj, lg, [10, 11, 12])
    assert oracle.graft_retrieve(adj, [10], [-1, 0, 1], [0, 0, 0])[0].tolist() == [11, 12, 13]


# ---------------------------------------------------------------------------
# Stochastic tree verification (recursive rejection sampling; the pages run at
# T = 1 -- BlockPilot §五, D-cut §4 -- and fix the one-token rule, SpecOPD
# §03.2). The defining property of speculative sampling is that the emitted
# tokens follow the target's distributions whatever the draft was; the pins
# check that property by sampling, the greedy limit against the C oracle,
# and closed forms.

def _chi2(counts, probs):
    counts = np.asarray(counts, np.float64)
    exp = probs * counts.sum()
    keep = exp > 0
    assert np.all(counts[~keep] == 0)
    return float(((counts[keep] - exp[keep]) ** 2 / exp[keep]).sum())


def _rrs_trials(rng, n_trials, v=6, width=(3, 2)):
    """Trees drawn the way a draft model draws them: the root's children are
    `width[0]` distinct tokens sampled from the draft's q at the root without
    replacement, each child's children `width[1]` tokens from q at that child.
    The target's and the draft's next-token logits depend on the token a node
    carries (a toy model with one step of context)."""
    t_root, d_root = rng.normal(0, 1.2, v), rng.normal(0, 1.2, v)
    t_tok, d_tok = rng.normal(0, 1.2, (v, v)), rng.normal(0, 1.2, (v, v))
    q_root = np.exp(d_root) / np.exp(d_root).sum()
    q_tok = np.exp(d_tok) / np.exp(d_tok).sum(1, keepdims=True)
    par, tok, tl, dl, cu = [], [], [], [], [0]
    for _ in range(n_trials):
        kids = rng.choice(v, size=width[0], replace=False, p=q_root)
        nodes = [(-1, 0, t_root, d_root)]
        for a in kids:
            nodes.append((0, int(a), t_tok[a], d_tok[a]))
        for ci, a in enumerate(kids):
            for g in rng.choice(v, size=width[1], replace=False, p=q_tok[a]):
                nodes.append((1 + ci, int(g), t_tok[g], d_tok[g]))
        for pp, tk, t, d in nodes:
            par.append(pp)
            tok.append(tk)
            tl.append(t)
            dl.append(d)
        cu.append(len(par))
    n = len(par)
    return (np.array(par, np.int32), np.array(tok, np.int32), np.array(cu, np.int32),
            np.array(tl), np.array(dl), rng.random(n), rng.random(n_trials), t_root, t_tok)


def _first_two_tokens(tok, cu, al, path, bonus):
    first, second = [], []
    for b in range(len(cu) - 1):
        lo = cu[b]
        toks = [tok[lo + path[b, d]] for d in range(1, al[b] + 1)] + [bonus[b]]
        first.append(toks[0])
        second.append(toks[1] if al[b] >= 1 else -1)
    return np.array(first), np.array(second)


def test_sampled_emitted_tokens_follow_the_target():
    rng = np.random.default_rng(31)
    v, n = 6, 12000
    par, tok, cu, tl, dl, ua, ub, t_root, t_tok = _rrs_trials(rng, n, v)
    al, path, bonus, _ = oracle.accept_sampled(par, tok, cu, tl, dl, 1.0, ua, ub, max_depth=2)
    first, second = _first_two_tokens(tok, cu, al, path, bonus)
    p_root = np.exp(t_root) / np.exp(t_root).sum()
    # 5 degrees of freedom: 40 is far beyond the 1e-6 quantile (35.9)
    assert _chi2(np.bincount(first, minlength=v), p_root) < 40
    # after an accepted child carrying token a, the next token follows the
    # target's distribution at that child
    tested = 0
    for a in range(v):
        sel = (al >= 1) & (first == a)
        if sel.sum() < 400:
            continue
        p_a = np.exp(t_tok[a]) / np.exp(t_tok[a]).sum()
        assert _chi2(np.bincount(second[sel], minlength=v), p_a) < 40, a
        tested += 1
    assert tested >= 3


def test_sampled_reduces_to_greedy_acceptance_as_temperature_vanishes(oracle_lib):
    rng = np.random.default_rng(32)
    v, batch = 40, 30
    par, tok, cu = [], [], [0]
    for b in range(batch):
        n = int(rng.integers(1, 24))
        p = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        t = [int(rng.integers(0, v))]
        for i in range(1, n):             # siblings carry distinct tokens
            used = {t[j] for j in range(1, i) if p[j] == p[i]}
            t.append(int(rng.choice([x for x in range(v) if x not in used])))
        par += p
        tok += t
        cu.append(len(par))
    n = len(par)
    tl = rng.normal(0, 3, (n, v))
    dl = rng.normal(0, 3, (n, v))
    # make many children agree with the target's argmax so that paths go deep
    for b in range(batch):
        lo, hi = cu[b], cu[b + 1]
        for c in range(lo + 1, hi):
            if rng.random() < 0.6:
                tl[lo + par[c], tok[c]] = tl[lo + par[c]].max() + 1.0
    target_tok = tl.argmax(1).astype(np.int32)
    al_g, path_g, bonus_g = oracle.accept(par, tok, target_tok, cu, max_depth=24)
    al, path, bonus, _ = oracle.accept_sampled(par, tok, cu, tl, dl, 1e-6, rng.random(n),
                                               rng.random(batch), max_depth=24)
    np.testing.assert_array_equal(al, al_g)
    np.testing.assert_array_equal(path, path_g)
    np.testing.assert_array_equal(bonus, bonus_g)
    assert al.max() >= 3


def test_sampled_one_child_is_accepted_with_probability_min_1_p_over_q():
    # two tokens: p = (a, 1-a), q = (c, 1-c); the root's one child carries
    # token 0. Over a grid of uniforms it is accepted for a fraction
    # min(1, a/c) of them; on rejection the residual is all on token 1.
    for a, c in ((0.3, 0.6), (0.6, 0.3), (0.25, 0.25)):
        grid = (np.arange(1000) + 0.5) / 1000
        n = len(grid)
        par = np.tile([-1, 0], n).astype(np.int32)
        tok = np.tile([5, 0], n).astype(np.int32)
        cu = np.arange(0, 2 * n + 1, 2).astype(np.int32)
        tl = np.tile([[np.log(a), np.log(1 - a)], [0.0, 0.0]], (n, 1))
        dl = np.tile([[np.log(c), np.log(1 - c)], [0.0, 0.0]], (n, 1))
        ua = np.zeros(2 * n)
        ua[1::2] = grid
        al, path, bonus, _ = oracle.accept_sampled(par, tok, cu, tl, dl, 1.0, ua,
                                                   np.full(n, 0.5), max_depth=1)
        assert abs(al.mean() - min(1.0, a / c)) <= 1.5e-3
        assert np.all(bonus[al == 0] == 1)        # residual max(0, p - q) sits on token 1
        assert np.all(path[al == 1, 1] == 1)


def test_sampled_bonus_is_inverse_transform_sampling():
    # a lone root: the bonus is drawn from p; over a uniform grid of K points
    # token v comes up K * p(v) times, up to one point per boundary
    rng = np.random.default_rng(33)
    v, k = 9, 3000
    logits = rng.normal(0, 1.5, v)
    logits[4] = -np.inf                        # a token with no mass is never drawn
    p = np.exp(logits - logits.max())
    p /= p.sum()
    grid = (np.arange(k) + 0.5) / k
    par = np.full(k, -1, np.int32)
    cu = np.arange(k + 1, dtype=np.int32)
    al, _, bonus, _ = oracle.accept_sampled(par, np.zeros(k, np.int32), cu, np.tile(logits, (k, 1)),
                                            np.zeros((k, v)), 1.0, np.zeros(k), grid, max_depth=0)
    assert np.all(al == 0)
    counts = np.bincount(bonus, minlength=v)
    assert counts[4] == 0
    assert np.all(np.abs(counts - k * p) <= 1.0 + 1e-9)
    assert np.all(np.diff(bonus) >= 0)         # token order: the grid is increasing


def test_sampled_draft_equal_to_target_takes_every_first_child():
    # q = p: every tried child has ratio 1, so the first child is always taken
    rng = np.random.default_rng(34)
    v = 12
    par = np.array([-1, 0, 0, 1, 1, 3, 2], np.int32)
    tok = np.array([0, 3, 4, 5, 6, 7, 8], np.int32)
    tl = rng.normal(0, 1, (7, v))
    tl[5] = -30.0
    tl[5, 9] = 30.0                            # the leaf's target is sure of token 9
    ua = rng.random(7) * 0.999
    al, path, bonus, _ = oracle.accept_sampled(par, tok, [0, 7], tl, tl.copy(), 1.0, ua, [0.7],
                                               max_depth=4)
    assert al[0] == 3 and path[0].tolist() == [0, 1, 3, 5, -1] and bonus[0] == 9


def test_sampled_temperature_scales_the_logits_and_bad_tokens_are_skipped():
    rng = np.random.default_rng(35)
    par, tok, cu, tl, dl, ua, ub, _, _ = _rrs_trials(rng, 200, 8)
    a = oracle.accept_sampled(par, tok, cu, tl, dl, 0.7, ua, ub, max_depth=2)
    b = oracle.accept_sampled(par, tok, cu, tl / 0.7, dl / 0.7, 1.0, ua, ub, max_depth=2)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)
    # children whose token is outside the vocabulary are passed over: with
    # every root child out of range the result is that of a lone root
    bad = tok.copy()
    kids = np.where(par == 0)[0]
    bad[kids] = -1
    bad[kids[::2]] = 8
    al, _, bonus, _ = oracle.accept_sampled(par, bad, cu, tl, dl, 1.0, ua, ub, max_depth=2)
    roots = cu[:-1]
    al1, _, bonus1, _ = oracle.accept_sampled(np.full(len(roots), -1, np.int32), tok[roots],
                                              np.arange(len(roots) + 1, dtype=np.int32),
                                              tl[roots], dl[roots], 1.0, ua[roots], ub, max_depth=0)
    assert np.all(al == 0) and np.all(al1 == 0)
    np.testing.assert_array_equal(bonus, bonus1)
