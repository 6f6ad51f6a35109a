"""GPU parity of tree_mask_build and tree_accept against the oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv
import workloads as W
from tv_testlib import Dev, mask_bits_u64

pytestmark = pytest.mark.gpu


def _pack(trees):
    cu = np.concatenate([[0], np.cumsum([len(t) for t in trees])]).astype(np.int32)
    par = np.concatenate([np.asarray(t, np.int32) for t in trees])
    return par, cu


def _gpu_bits(par, cu, max_nodes, words):
    m = tv.tree_mask_build(torch.from_numpy(par).cuda(), torch.from_numpy(cu).cuda(), max_nodes,
                           kind="bits", words_per_node=words)
    return mask_bits_u64(m["bits"]), m["depth"].cpu().numpy(), m["err"].cpu().numpy()


def _gpu_anchor(par, cu, max_nodes):
    m = tv.tree_mask_build(torch.from_numpy(par).cuda(), torch.from_numpy(cu).cuda(), max_nodes,
                           kind="anchor")
    return (m["anchor_pos"].cpu().numpy(), m["branch_depth"].cpu().numpy(),
            m["depth"].cpu().numpy(), m["err"].cpu().numpy())


@pytest.mark.parametrize("sizes,words", [
    ([15], 1), ([60], 1), ([1, 2, 63, 64], 1), ([65, 100, 128], 2), ([300, 17, 1], 5),
    ([1024, 999], 16), ([513], 9),
])
def test_mask_bits_random_trees(sizes, words):
    rng = np.random.default_rng(sum(sizes) + words)
    trees = [W.random_tree(rng, n, max_children=int(rng.integers(1, 5))) for n in sizes]
    par, cu = _pack(trees)
    bits, depth, err = _gpu_bits(par, cu, max(sizes), words)
    obits, odepth, oerr = oracle.mask_bits(par, cu, words)
    np.testing.assert_array_equal(err, oerr)
    np.testing.assert_array_equal(bits, obits)
    np.testing.assert_array_equal(depth, odepth)


def test_mask_bits_chain_and_star_at_the_word_limit():
    chain = [-1] + list(range(1023))
    star = [-1] + [0] * 1023
    par, cu = _pack([chain, star])
    bits, depth, err = _gpu_bits(par, cu, 1024, 16)
    obits, odepth, oerr = oracle.mask_bits(par, cu, 16)
    np.testing.assert_array_equal(bits, obits)
    np.testing.assert_array_equal(depth, odepth)
    assert err.tolist() == [0, 0]


def test_mask_bits_config_trees():
    for c in (1, 2):
        w = W.make(c, prefix=16)
        bits, depth, err = _gpu_bits(w.parent, w.cu_nodes, w.max_nodes, w.words_per_node)
        obits, odepth, oerr = oracle.mask_bits(w.parent, w.cu_nodes, w.words_per_node)
        np.testing.assert_array_equal(bits, obits)
        np.testing.assert_array_equal(depth, odepth)
    w = W.make(3, batch=64, prefix_range=(1, 2))
    bits, depth, err = _gpu_bits(w.parent, w.cu_nodes, w.max_nodes, 1)
    obits, odepth, oerr = oracle.mask_bits(w.parent, w.cu_nodes, 1)
    np.testing.assert_array_equal(bits, obits)
    np.testing.assert_array_equal(depth, odepth)


@pytest.mark.parametrize("bad", [[0, 0, 1], [-1, 0, 2], [-1, 0, 3, 1], [-1, 0, -1], [-1, -2, 0]])
def test_mask_reports_malformed_trees(bad):
    good = [-1, 0, 0, 1]
    par, cu = _pack([good, bad, good])
    bits, depth, err = _gpu_bits(par, cu, 4, 1)
    obits, odepth, oerr = oracle.mask_bits(par, cu, 1)
    assert err.tolist() == oerr.tolist() == [0, 1, 0]
    np.testing.assert_array_equal(bits, obits)
    np.testing.assert_array_equal(depth, odepth)
    ap, bd, d2, err2 = _gpu_anchor(par, cu, 4)
    oap, obd, od2, oerr2 = oracle.mask_anchor(par, cu)
    np.testing.assert_array_equal(err2, oerr2)
    np.testing.assert_array_equal(ap, oap)
    np.testing.assert_array_equal(bd, obd)
    np.testing.assert_array_equal(d2, od2)


def test_mask_bits_too_many_nodes_for_words_sets_err():
    chain = [-1] + list(range(99))
    par, cu = _pack([chain, [-1, 0]])
    # words=1 cannot hold 100 nodes: the host check refuses a max_nodes above 64
    with pytest.raises(tv.TVError):
        _gpu_bits(par, cu, 100, 1)
    # a max_nodes that understates the tree: the device reports it per request
    bits, depth, err = _gpu_bits(par, cu, 64, 1)
    assert err.tolist() == [1, 0]
    assert (bits[:100] == 0).all() and (depth[:100] == -1).all()


@pytest.mark.parametrize("seed", range(4))
def test_mask_anchor_random_trunk_branch(seed):
    rng = np.random.default_rng(seed)
    trees = []
    for _ in range(5):
        trunk = int(rng.integers(1, 700))
        nb = int(rng.integers(0, 40))
        anchors = np.sort(rng.integers(0, trunk, size=nb)).tolist()
        trees.append(W.trunk_branch_tree(trunk, anchors, int(rng.integers(1, 24))))
    bad = W.trunk_branch_tree(50, [10, 20], 5)
    bad.append(len(bad) - 2)                       # branch of a branch
    trees.append(bad)
    par, cu = _pack(trees)
    ap, bd, depth, err = _gpu_anchor(par, cu, max(len(t) for t in trees))
    oap, obd, odepth, oerr = oracle.mask_anchor(par, cu)
    assert err.tolist() == oerr.tolist() and oerr[-1] == 2
    np.testing.assert_array_equal(ap, oap)
    np.testing.assert_array_equal(bd, obd)
    np.testing.assert_array_equal(depth, odepth)


def test_mask_anchor_specopd_tree():
    w = W.make(5)
    ap, bd, depth, err = _gpu_anchor(w.parent, w.cu_nodes, w.max_nodes)
    oap, obd, odepth, oerr = oracle.mask_anchor(w.parent, w.cu_nodes)
    assert err.tolist() == [0]
    np.testing.assert_array_equal(ap, oap)
    np.testing.assert_array_equal(bd, obd)
    np.testing.assert_array_equal(depth, odepth)


def test_mask_anchor_request_sizes_around_the_staged_limit():
    """ANCHOR requests of up to 8192 nodes are read into LDS at once; exactly
    8192 nodes (trunk 8128 + 4 branches of 16) and, with a larger max_nodes,
    8660 nodes (trunk 8500 + 10 branches of 16, the strided kernel) match the
    oracle; a request past 8192 nodes under a max_nodes of 8192 (the caller
    understating it) is reported malformed while its neighbour is exact."""
    rng = np.random.default_rng(8192)
    t8192 = W.trunk_branch_tree(8128, np.sort(rng.integers(0, 8128, size=4)).tolist(), 16)
    t8660 = W.trunk_branch_tree(8500, np.sort(rng.integers(0, 8500, size=10)).tolist(), 16)
    small = W.trunk_branch_tree(40, [3, 17, 17], 5)
    assert len(t8192) == 8192 and len(t8660) == 8660
    for trees, max_nodes in (([t8192, small], 8192), ([small, t8660, t8192], 8660)):
        par, cu = _pack(trees)
        ap, bd, depth, err = _gpu_anchor(par, cu, max_nodes)
        oap, obd, odepth, oerr = oracle.mask_anchor(par, cu)
        assert err.tolist() == oerr.tolist() == [0] * len(trees)
        np.testing.assert_array_equal(ap, oap)
        np.testing.assert_array_equal(bd, obd)
        np.testing.assert_array_equal(depth, odepth)
    par, cu = _pack([t8660, small])
    ap, bd, depth, err = _gpu_anchor(par, cu, 8192)
    oap, obd, odepth, oerr = oracle.mask_anchor(par, cu)
    assert err.tolist() == [1, 0]
    assert (ap[:8660] == -1).all() and (bd[:8660] == 0).all() and (depth[:8660] == -1).all()
    np.testing.assert_array_equal(ap[8660:], oap[8660:])
    np.testing.assert_array_equal(bd[8660:], obd[8660:])
    np.testing.assert_array_equal(depth[8660:], odepth[8660:])


# -------------------------------------------------------------- acceptance --

def _check_accept(w, max_depth=None):
    d = Dev(w)
    md = w.max_depth if max_depth is None else max_depth
    al, path, bonus = d.accept(md)
    oal, opath, obonus = oracle.accept(w.parent, w.draft_tok, w.target_tok, w.cu_nodes, md)
    np.testing.assert_array_equal(al.cpu().numpy(), oal)
    np.testing.assert_array_equal(path.cpu().numpy(), opath)
    np.testing.assert_array_equal(bonus.cpu().numpy(), obonus)
    return oal


@pytest.mark.parametrize("config", [1, 2, 3, 4])
def test_accept_config_workloads(config):
    kw = {1: {}, 2: {"prefix": 16}, 3: {"prefix_range": (1, 2)}, 4: {"prefix": 16}}[config]
    w = W.make(config, **kw)
    al = _check_accept(w)
    if w.batch > 1:
        assert al.max() > 0      # batches of generated trees accept something


@pytest.mark.parametrize("sizes,vocab", [([1, 2, 3], 3), ([64, 65, 129], 4), ([700, 2000], 3),
                                         ([8192], 2), ([63, 1, 200], 40)])
def test_accept_random_trees(sizes, vocab):
    rng = np.random.default_rng(len(sizes) * 1000 + vocab)
    trees = [W.random_tree(rng, n, max_children=int(rng.integers(1, 6))) for n in sizes]
    w = W.build_workload("acc", trees, [0] * len(trees), 2, 1, 8, "f32", rng, vocab=vocab,
                         match_p=0.9)
    _check_accept(w)
    _check_accept(w, max_depth=3)          # path rows shorter than the best path


def test_accept_chains_and_repeated_siblings():
    trees = [[-1] + list(range(15))] * 6 + [[-1, 0, 0, 2, 1]]
    w = W.build_workload("acc", trees, [0] * len(trees), 2, 1, 8, "f32", 5, vocab=2, match_p=0.6)
    w.draft_tok[-5:] = [0, 7, 7, 9, 9]
    w.target_tok[-5:] = [7, 9, 9, 0, 0]
    al = _check_accept(w)
    assert al[-1] == 2


def test_accept_empty_requests_first_middle_last():
    """Requests with no nodes (first, in the middle, twice in a row, last):
    accept_len 0, path all -1, bonus -1; the others match the oracle."""
    rng = np.random.default_rng(5)
    trees = [W.random_tree(rng, n) for n in (7, 1, 30, 100)]
    for layout in ([None, 0, 1], [0, None, None, 2], [3, 1, None], [None]):
        sub = [trees[k] if k is not None else [] for k in layout]
        par, cu = _pack(sub)
        dr = rng.integers(4, size=len(par)).astype(np.int32)
        tg = rng.integers(4, size=len(par)).astype(np.int32)
        dev = "cuda"
        if len(par) == 0:
            par, dr, tg = np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(1, np.int32)
        al, path, bonus = tv.tree_accept(torch.from_numpy(par).to(dev), torch.from_numpy(dr).to(dev),
                                         torch.from_numpy(tg).to(dev), torch.from_numpy(cu).to(dev),
                                         128, 12)
        oal, opath, obonus = oracle.accept(par, dr, tg, cu, 12)
        np.testing.assert_array_equal(al.cpu().numpy(), oal)
        np.testing.assert_array_equal(path.cpu().numpy(), opath)
        np.testing.assert_array_equal(bonus.cpu().numpy(), obonus)
        for b, k in enumerate(layout):
            if k is None:
                assert oal[b] == 0 and obonus[b] == -1 and (opath[b] == -1).all()

