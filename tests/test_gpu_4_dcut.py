"""GPU parity of tv_dcut_select against the oracle: every output bit-exact
(the kept lengths are integer decisions taken on fp32 scores formed the same
way on both sides). Shapes: the config-3 batch (64 x 15) over the budget-ratio
grid, exact ties, out-of-range confidences, one request, more requests than
threads, the position limit, and the packed trees fed to tree_mask_build."""
import numpy as np
import pytest
import torch

import oracle
import tree_verification_attention_mask_amd as tv
import workloads as W

pytestmark = pytest.mark.gpu


def _gpu(conf, tokens, budget):
    c = torch.from_numpy(np.ascontiguousarray(conf, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
    n, cu, par, tok = tv.dcut_select(c, t, budget)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (n, cu, par, tok)]


def _check(conf, budget, seed=0, what=""):
    conf = np.asarray(conf, np.float32)
    b, d = conf.shape
    tokens = np.random.default_rng(seed).integers(0, 151936, size=(b, d + 1)).astype(np.int32)
    got = _gpu(conf, tokens, budget)
    ref = oracle.dcut_select(conf, tokens, budget)
    for name, g, r in zip(("n_keep", "cu_nodes", "parent", "packed_tokens"), got, ref):
        np.testing.assert_array_equal(g, r, err_msg="%s %s budget=%d" % (what, name, budget))
    return got


@pytest.mark.parametrize("rho", [0.25, 0.5, 0.75, 1.0])
def test_config3_batch_over_the_budget_grid(rho):
    rng = np.random.default_rng(3)
    conf = rng.beta(4.0, 2.0, size=(64, 15))
    budget = int(round(rho * 64 * 16))
    n = _check(conf, budget, what="rho=%g" % rho)[0]
    assert n.sum() == budget


def test_config3_recipe_lengths():
    w = W.make(3)
    n = _check(np.asarray(w.meta["confidence"], np.float32), w.meta["budget"])[0]
    assert n.tolist() == [int(x) for x in w.nodes_per_request]


@pytest.mark.parametrize("budget", [64, 65, 100, 500, 1023, 1024])
def test_every_budget_edge(budget):
    rng = np.random.default_rng(budget)
    _check(rng.uniform(0, 1, size=(64, 15)), budget, seed=budget)


def test_exact_ties_go_to_smaller_requests_then_positions():
    rng = np.random.default_rng(5)
    conf = rng.choice(np.array([0.5, 0.25, 1.0, 0.0], np.float32), size=(50, 9))
    for budget in (50, 61, 137, 200, 333, 500):
        _check(conf, budget, what="ties")
    _check(np.full((33, 7), 0.5, np.float32), 33 + 70, what="all equal")


def test_confidences_outside_the_unit_interval():
    rng = np.random.default_rng(6)
    conf = rng.uniform(-0.5, 1.5, size=(40, 12)).astype(np.float32)
    conf[rng.random(conf.shape) < 0.05] = np.nan
    conf[0, :] = np.inf
    for budget in (40, 120, 300, 520):
        _check(conf, budget, what="clamped")


@pytest.mark.parametrize("batch,d", [(1, 1), (1, 63), (3, 2), (1025, 3), (2048, 15), (32768, 1),
                                     (512, 64)])
def test_shapes_up_to_the_position_limit(batch, d):
    rng = np.random.default_rng(batch + d)
    conf = rng.beta(4.0, 2.0, size=(batch, d))
    for frac in (0.0, 0.3, 1.0):
        budget = batch + int(round(frac * batch * d))
        _check(conf, budget, seed=batch, what="%dx%d" % (batch, d))


def test_limits_are_refused():
    c = torch.zeros((2049, 16), dtype=torch.float32, device="cuda")
    t = torch.zeros((2049, 17), dtype=torch.int32, device="cuda")
    with pytest.raises(tv.TVError) as e:
        tv.dcut_select(c, t, 2049)
    assert e.value.status == 2
    c2 = torch.zeros((4, 3), dtype=torch.float32, device="cuda")
    t2 = torch.zeros((4, 4), dtype=torch.int32, device="cuda")
    for bad in (3, 17):
        with pytest.raises(tv.TVError) as e:
            tv.dcut_select(c2, t2, bad)
        assert e.value.status == 1


def test_packed_chains_feed_tree_mask_build():
    rng = np.random.default_rng(8)
    conf = rng.beta(4.0, 2.0, size=(64, 15)).astype(np.float32)
    tokens = rng.integers(0, 1000, size=(64, 16)).astype(np.int32)
    c = torch.from_numpy(conf).cuda()
    t = torch.from_numpy(tokens).cuda()
    n, cu, par, tok = tv.dcut_select(c, t, 512)
    m = tv.tree_mask_build(par, cu, 16, kind="bits", words_per_node=1)
    torch.cuda.synchronize()
    obits, odepth, oerr = oracle.mask_bits(par.cpu().numpy(), cu.cpu().numpy(), 1)
    assert (m["err"].cpu().numpy() == 0).all() and (oerr == 0).all()
    np.testing.assert_array_equal(m["bits"].cpu().numpy().view(np.uint64), obits)
    np.testing.assert_array_equal(m["depth"].cpu().numpy(), odepth)
