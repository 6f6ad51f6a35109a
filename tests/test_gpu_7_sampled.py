"""GPU parity of tv_tree_accept_sampled (recursive rejection sampling) against
the oracle (float64 numpy), plus the defining property on the device itself.

Bar: accept_len, path and bonus token are integers and must match exactly.
The decisions are taken on floats -- u * q(x) < p(x) for a child, the
inverse-transform draw for the bonus -- in fp32 on the device and in float64
in the oracle, so a uniform within rounding of its threshold may legitimately
go either way. The oracle reports each request's smallest decision margin;
a request may differ only when that margin is below 1e-4 (fp32 softmax values
carry ~1e-6 relative error; a residual's normaliser and a bonus run's prefix
sums over 1.5e5 terms stay within ~1e-5), and such ties must stay rare.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv
import workloads as W

pytestmark = pytest.mark.gpu

TIE = 1e-4


def _run(si, dtype=torch.bfloat16, temperature=1.0, max_depth=None, offset=0, max_nodes=None):
    dev = "cuda"
    n, v = si.target_logits.shape
    if offset:   # rows that do not start on a 16-byte boundary
        bt = torch.empty(n * v + offset, dtype=dtype, device=dev)
        bd = torch.empty(n * v + offset, dtype=dtype, device=dev)
        bt[offset:] = torch.from_numpy(si.target_logits).to(dtype).reshape(-1).to(dev)
        bd[offset:] = torch.from_numpy(si.draft_logits).to(dtype).reshape(-1).to(dev)
        tl, dl = bt[offset:].view(n, v), bd[offset:].view(n, v)
    else:
        tl = torch.from_numpy(si.target_logits).to(dtype).to(dev)
        dl = torch.from_numpy(si.draft_logits).to(dtype).to(dev)
    md = si.max_depth if max_depth is None else max_depth
    sizes = np.diff(si.cu_nodes)
    mn = int(sizes.max()) if max_nodes is None else max_nodes
    al, path, bonus = tv.tree_accept_sampled(
        torch.from_numpy(si.parent).to(dev), torch.from_numpy(si.draft_tok).to(dev),
        torch.from_numpy(si.cu_nodes).to(dev), tl, dl, torch.from_numpy(si.u_accept).to(dev),
        torch.from_numpy(si.u_bonus).to(dev), max(mn, 1), max(si.max_children, 1), md,
        temperature)
    torch.cuda.synchronize()
    ref = oracle.accept_sampled(si.parent, si.draft_tok, si.cu_nodes, tl.float().cpu().numpy(),
                                dl.float().cpu().numpy(), temperature, si.u_accept, si.u_bonus,
                                md)
    return (al.cpu().numpy(), path.cpu().numpy(), bonus.cpu().numpy()), ref


def _compare(got, ref, max_ties=1):
    al, path, bonus = got
    ral, rpath, rbonus, margin = ref
    diff = (al != ral) | (bonus != rbonus) | np.any(path != rpath, axis=1)
    ties = 0
    for b in np.nonzero(diff)[0]:
        assert margin[b] < TIE, (b, al[b], ral[b], bonus[b], rbonus[b], margin[b])
        ties += 1
    assert ties <= max_ties, ties
    return int((~diff).sum())


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_graft_tree_full_vocabulary(seed):
    # the 60-slot Graft tree, Qwen3's 151,936-token vocabulary, bf16 logits;
    # children drawn from the draft without replacement
    rng = np.random.default_rng(100 + seed)
    si = W.sampled_inputs(rng, [list(W.GRAFT_TREE_PARENT)] * 4, W.QWEN3_VOCAB)
    got, ref = _run(si)
    assert _compare(got, ref) >= 3
    assert got[0].max() >= 1


def test_benchmark_input_and_launch():
    # the exact input and launch shape bench.py times: one Graft tree, seed 2,
    # 151,936-token bf16 logits (10 shares per row)
    si = W.sampled_inputs(np.random.default_rng(2), [list(W.GRAFT_TREE_PARENT)], W.QWEN3_VOCAB)
    got, ref = _run(si)
    _compare(got, ref, max_ties=0)
    assert got[0][0] >= 1


@pytest.mark.parametrize("temperature", [0.6, 1.0, 1.7])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_small_trees_many_requests(temperature, dtype):
    rng = np.random.default_rng(int(temperature * 10) + (dtype == torch.float32))
    trees = [W.random_tree(rng, int(rng.integers(1, 40)), max_children=6) for _ in range(48)]
    si = W.sampled_inputs(rng, trees, 1000, dtype=dtype, spread=2.0, noise=0.7,
                          temperature=temperature)
    got, ref = _run(si, dtype=dtype, temperature=temperature)
    assert _compare(got, ref, max_ties=2) >= 46


def test_many_requests_and_the_per_level_walk():
    # 256 requests (one share per row: the walk reads a node per level when
    # the request's tables do not fit its LDS), bf16, 4096-token vocabulary
    rng = np.random.default_rng(44)
    trees = [W.random_tree(rng, int(rng.integers(1, 31)), max_children=8) for _ in range(256)]
    si = W.sampled_inputs(rng, trees, 4096, dtype=torch.bfloat16, spread=2.5, noise=0.8)
    got, ref = _run(si)
    assert _compare(got, ref, max_ties=3) >= 250
    # the same batch with a node cap too large for the walk's LDS tables
    got2, _ = _run(si, max_nodes=8192)
    for x, y in zip(got, got2):
        np.testing.assert_array_equal(x, y)


def test_matches_greedy_acceptance_as_temperature_vanishes():
    rng = np.random.default_rng(7)
    trees = [W.random_tree(rng, int(rng.integers(2, 30)), max_children=5) for _ in range(32)]
    v = 500
    si = W.sampled_inputs(rng, trees, v, dtype=torch.float32, spread=4.0)
    # distinct logits 0.05 apart: at T = 1e-4 both softmaxes are exactly one-hot
    # (the next value is 2^-721 below), in fp32 and in float64
    n = len(si.parent)
    si.target_logits = np.stack([rng.permutation(v) * 0.05 for _ in range(n)]).astype(np.float32)
    si.draft_logits = np.stack([rng.permutation(v) * 0.05 for _ in range(n)]).astype(np.float32)
    # make most children agree with the target's argmax so that paths go deep
    for b in range(len(trees)):
        lo, hi = si.cu_nodes[b], si.cu_nodes[b + 1]
        for c in range(lo + 1, hi):
            if rng.random() < 0.6:
                row = si.target_logits[lo + si.parent[c]]
                row[si.draft_tok[c]] = row.max() + 1.0
    target_tok = si.target_logits.argmax(1).astype(np.int32)
    got, ref = _run(si, dtype=torch.float32, temperature=1e-4)
    gal, gpath, gbonus = oracle.accept(si.parent, si.draft_tok, target_tok, si.cu_nodes,
                                       si.max_depth)
    np.testing.assert_array_equal(got[0], gal)
    np.testing.assert_array_equal(got[1], gpath)
    np.testing.assert_array_equal(got[2], gbonus)
    dal, dpath, dbonus = tv.tree_accept(
        torch.from_numpy(si.parent).cuda(), torch.from_numpy(si.draft_tok).cuda(),
        torch.from_numpy(target_tok).cuda(), torch.from_numpy(si.cu_nodes).cuda(),
        int(np.diff(si.cu_nodes).max()), si.max_depth)
    np.testing.assert_array_equal(got[0], dal.cpu().numpy())
    np.testing.assert_array_equal(got[2], dbonus.cpu().numpy())
    assert got[0].max() >= 3


def test_emitted_tokens_follow_the_target_on_the_device():
    # 6000 independent trials of a small tree drawn from the draft: the first
    # emitted token (accepted child or bonus) must follow the target at the
    # root, whatever the draft was (chi-square, 7 degrees of freedom)
    rng = np.random.default_rng(8)
    v, trials = 8, 6000
    t_root = rng.normal(0, 1.2, v).astype(np.float32)
    d_root = rng.normal(0, 1.2, v).astype(np.float32)
    tree = [-1, 0, 0, 0, 1, 1, 2]
    si = W.sampled_inputs(rng, [tree] * trials, v, dtype=torch.float32, spread=1.2, noise=1.0)
    # every trial shares the root's distributions; redraw the root's children
    # from that draft (without replacement) so the trials are identically distributed
    q = np.exp(d_root.astype(np.float64))
    q /= q.sum()
    for b in range(trials):
        lo = si.cu_nodes[b]
        si.target_logits[lo] = t_root
        si.draft_logits[lo] = d_root
        si.draft_tok[lo + 1: lo + 4] = rng.choice(v, size=3, replace=False, p=q)
    got, ref = _run(si, dtype=torch.float32)
    _compare(got, ref, max_ties=3)
    al, path, bonus = got
    first = np.where(al >= 1, si.draft_tok[si.cu_nodes[:-1] + np.maximum(path[:, 1], 0)], bonus)
    p = np.exp(t_root.astype(np.float64))
    p /= p.sum()
    counts = np.bincount(first, minlength=v)
    chi2 = float(((counts - trials * p) ** 2 / (trials * p)).sum())
    assert chi2 < 45, (chi2, counts, trials * p)


def test_edge_cases():
    rng = np.random.default_rng(9)
    v = 777   # not a multiple of 8: one value per load
    trees = [[-1], [-1, 0, 0, 1], [-1] + [0] * 40, [-1, 0, 1, 2, 3, 4, 5]]
    si = W.sampled_inputs(rng, trees, v, dtype=torch.bfloat16)
    lo = si.cu_nodes
    si.draft_tok[lo[1] + 2] = -5                 # outside the vocabulary: passed over
    si.draft_tok[lo[1] + 3] = v + 3
    si.draft_tok[lo[2] + 7] = si.draft_tok[lo[2] + 6]   # a repeated sibling token
    si.u_accept[lo[2] + 1: lo[2] + 41] = 0.9999  # reject almost every child of the wide root
    si.target_logits[lo[3] + 2, :] = np.nan      # NaN logits count as -inf
    si.target_logits[lo[3] + 2, 5] = 1.0
    si.draft_logits[lo[3] + 3, : v // 2] = -np.inf
    si.draft_logits[lo[3] + 1, ::5] = np.nan     # NaN draft logits: no draft mass there
    si.draft_logits[lo[2], 1::3] = np.nan
    si.u_accept[lo[3] + 1: lo[3] + 7] = 0.0      # the chain is taken as far as mass allows
    got, ref = _run(si)
    _compare(got, ref, max_ties=0)
    got, ref = _run(si, offset=1)                # unaligned rows
    _compare(got, ref, max_ties=0)
    # an empty request, and a path row shorter than the tree's depth
    si2 = W.sampled_inputs(rng, [[-1, 0, 1, 2, 3]], 64, dtype=torch.float32, spread=0.1)
    si2.parent = np.concatenate([si2.parent, np.zeros(0, np.int32)])
    si2.cu_nodes = np.array([0, 0, 5], np.int32)
    si2.u_bonus = np.array([0.5, si2.u_bonus[0]], np.float32)
    si2.u_accept[:] = 0.0
    got, ref = _run(si2, dtype=torch.float32, max_depth=2)
    _compare(got, ref, max_ties=0)
    assert got[0][0] == 0 and got[2][0] == -1 and np.all(got[1][0] == -1)


def test_draft_equal_to_target_takes_first_children():
    rng = np.random.default_rng(10)
    si = W.sampled_inputs(rng, [list(W.GRAFT_TREE_PARENT)] * 3, 4096, dtype=torch.float32)
    si.draft_logits = si.target_logits.copy()
    si.u_accept[:] = np.minimum(si.u_accept, 0.999)
    got, ref = _run(si, dtype=torch.float32)
    _compare(got, ref, max_ties=0)
    # the first child of every node on the path is taken down to a leaf
    par = np.array(W.GRAFT_TREE_PARENT)
    node, depth = 0, 0
    while True:
        kids = np.nonzero(par == node)[0]
        if len(kids) == 0:
            break
        node, depth = int(kids[0]), depth + 1
    assert np.all(got[0] == depth)


def test_argument_checks():
    z = torch.zeros(4, dtype=torch.int32, device="cuda")
    f = torch.zeros(4, dtype=torch.float32, device="cuda")
    lg = torch.zeros((4, 10), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    ub = torch.zeros(1, dtype=torch.float32, device="cuda")
    for kw, status in (({"temperature": 0.0}, 1), ({"temperature": float("inf")}, 1),
                       ({"max_children": 100000}, 2), ({"max_nodes": 100000}, 2)):
        args = dict(max_nodes=4, max_children=3, max_depth=3, temperature=1.0)
        args.update(kw)
        with pytest.raises(tv.TVError) as e:
            tv.tree_accept_sampled(z, z, cu, lg, lg, f, ub, **args)
        assert e.value.status == status
